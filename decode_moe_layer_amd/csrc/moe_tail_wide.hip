// The wide kernels of the fused decode MoE layer tail: one launch of 17..32
// rows, with the kernel body of moe_tail_device.h.  A translation unit of
// their own, so that the narrow kernels' code object (moe_tail.hip) is laid
// out the same with or without them.
#include "moe_tail_device.h"

namespace mt {

// wide launches (17..32 rows), activations from global scratch
MT_KERNEL(moe_tail_kernel_gm_w, false, false, false, false, true)
MT_KERNEL(moe_tail_kernel_gm_wf, false, false, true, false, true)
MT_KERNEL(moe_tail_kernel_gm_w8, false, false, false, true, true)
MT_KERNEL(moe_tail_kernel_gm_wf8, false, false, true, true, true)
#undef MT_KERNEL

}  // namespace mt
