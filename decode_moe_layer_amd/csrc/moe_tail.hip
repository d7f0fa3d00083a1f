// Fused decode MoE layer tail for MI355X (gfx950): one persistent launch.
//
// Steps (one tensor-parallel rank's shard, 1..32 rows), after "[AMD]
// integrate kimi k3 monokernel" (sglang PR 43481), K2 commit text, sections
// Motivation and "Kernel Replacement":
//   norm    h = bf16(x + residual); xn = bf16(h * rstd * gamma), rstd in fp64
//   router  logits = xn . Wr^T (fp32)
//   top-k   K rounds of a wave-wide maximum, exact ties to the lower expert id
//           ("glm53: Long-context indexer ...", PR 85 commit row 9)
//   dedup   each distinct expert of the step is one slot with its using rows;
//           its weights stream from HBM once (PR 85 commit rows 16 and 20)
//   gate/up per (slot, 8 intermediate indices): 16 MFMA rows (8 gate + 8 up)
//           against all using rows as MFMA columns; a = silu(g) * u
//   shared  the bf16 shared expert's gate/up the same way
//   down    per workgroup a range of hidden rows: every slot's down tile and
//           the shared down tile, products kept per (pick, row) in LDS
//   combine y = sum over picks in (row, k) order of w * d, plus the shared
//           output, in fp32 and a fixed order; out = bf16(h + y)
//           (chunk-ordered fp32 partials: "Split the Kimi3 AttnRes mix across
//           CTAs for decode rows", flare PR 11, design section)
//
// A call of 17..32 rows runs as one wide launch (moe_tail_wide.hip): two
// 16-column MFMA tiles where rows are columns, one slot per 16 users of an
// expert, so experts are still de-duplicated across all rows; handles that
// cannot take it run such calls as narrow launches of at most 16 rows.  With
// attention rows in place of x, the out_proj front (K2 commit text,
// Motivation and Modifications) runs first in the same launch:
// x = bf16(attn . W_o^T), summed in double.
//
// Optional steps (separate kernel variants): the shared expert's output scaled
// by a sigmoid gate of the normed row (K2 commit text, Kernel Replacement), and
// group-limited routing with a routed scaling factor; and routed experts in
// MXFP8 (E4M3 codes, one byte each, with the same E8M0 block-32 scales; the
// FP8 expert path of PR 85, its commits on 16-byte FP8 loads and on the FP8
// mid).  An MXFP8 column group is two 16-byte lane loads instead of one,
// decoded with v_cvt_scalef32_pk_bf16_fp8, exact in bf16 like E2M1; the
// activations of the down projection stay bf16 (no FP8 re-quantisation of
// the mid, which would add error beyond the tail's tolerance).
//
// Cross-workgroup exchange goes through handle-owned scratch.  Every
// workgroup counts the calls it has started (its epoch).  On the router chain
// the data carry the epoch as a tag (xn chunks, router partials, logits), so
// a reader polls the data themselves; elsewhere counters in two banks,
// selected by the epoch's parity, release the readers, and no reset is needed
// between calls or graph replays.  Every wait has a deadline and a shared
// abort word (K2 commit text, Motivation: each wait has a deadline, a failed
// wait stops the launch everywhere; "Split the Kimi3 AttnRes mix across CTAs
// for decode rows", design section: per-call tags in the exchanged words).
//
// GEMV tiles use v_mfma_f32_16x16x32_bf16: weights are the A operand (16
// rows), activations the B operand (16 rows as columns per tile), staged in LDS.
// MXFP4 codes are dequantised exactly to bf16 with v_cvt_scalef32_pk_bf16_fp4
// (E2M1 x 2^(s-127) is exact in bf16 for the scales in range), so every
// product is exact and accumulation is fp32.  A lane's 16-byte weight load is
// one whole 32-element scale block (PR 85 commit row 18's 16-byte loads);
// weights are read once per call (the pages use nontemporal loads, commit
// row 21; here the default policy measured faster, see the buffer-access
// note below), and each wave keeps a deep window of them in flight, issued
// ahead of the waits they do not depend on (PR 85: weights are issued before
// an activation poll is checked).

#include <hip/hip_runtime.h>
#include <mutex>
#include <vector>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <type_traits>

#include "moe_tail.h"
#include "moe_tail_device.h"

namespace mt {

// The narrow kernels (the wide ones are in moe_tail_wide.hip).
MT_KERNEL(moe_tail_kernel_lds, true, false, false, false, false)
MT_KERNEL(moe_tail_kernel_lds_rs, true, true, false, false, false)
MT_KERNEL(moe_tail_kernel_gm, false, false, false, false, false)
MT_KERNEL(moe_tail_kernel_lds_f, true, false, true, false, false)
MT_KERNEL(moe_tail_kernel_lds_rs_f, true, true, true, false, false)
MT_KERNEL(moe_tail_kernel_gm_f, false, false, true, false, false)
// MXFP8 experts (E4M3 codes), without and with the optional steps
MT_KERNEL(moe_tail_kernel_lds_8, true, false, false, true, false)
MT_KERNEL(moe_tail_kernel_lds_rs_8, true, true, false, true, false)
MT_KERNEL(moe_tail_kernel_gm_8, false, false, false, true, false)
MT_KERNEL(moe_tail_kernel_lds_f8, true, false, true, true, false)
MT_KERNEL(moe_tail_kernel_lds_rs_f8, true, true, true, true, false)
MT_KERNEL(moe_tail_kernel_gm_f8, false, false, true, true, false)
#undef MT_KERNEL
static const void* kernel_for(const Params& p, bool wide) {
  const bool f = p.sgate || p.n_group > 1 || p.fold || p.attn;
  if (wide) {
    if (p.f8) return f ? (const void*)moe_tail_kernel_gm_wf8 : (const void*)moe_tail_kernel_gm_w8;
    return f ? (const void*)moe_tail_kernel_gm_wf : (const void*)moe_tail_kernel_gm_w;
  }
  if (p.f8) {
    if (!p.xn_lds) return f ? (const void*)moe_tail_kernel_gm_f8 : (const void*)moe_tail_kernel_gm_8;
    if (p.rsum) return f ? (const void*)moe_tail_kernel_lds_rs_f8 : (const void*)moe_tail_kernel_lds_rs_8;
    return f ? (const void*)moe_tail_kernel_lds_f8 : (const void*)moe_tail_kernel_lds_8;
  }
  if (!p.xn_lds) return f ? (const void*)moe_tail_kernel_gm_f : (const void*)moe_tail_kernel_gm;
  if (p.rsum) return f ? (const void*)moe_tail_kernel_lds_rs_f : (const void*)moe_tail_kernel_lds_rs;
  return f ? (const void*)moe_tail_kernel_lds_f : (const void*)moe_tail_kernel_lds;
}

}  // namespace mt

// ==================================================================== host ==

// Dynamic LDS plan.  The router/shared phase stages its K chunk of xn
// [rows][H/S1 + pad]; the routed gate/up phase then stages all of xn
// [rows][H + pad] when it fits; the down phase (which reuses the same space)
// stages the routed a [picks][I + pad], the shared a [rows][Is + pad], the
// per-pick products [picks][HR] and the shared partials [waves][rows][HR].
struct LdsPlan {
  int xn_lds, xs, cs, as, ss, off_as, off_outp, off_shp;
  int pa;  // routed a rows the down phase stages at once (all of them, except in a wide launch)
  size_t down, xn, chunk, dyn;
};

static size_t al16(size_t n) { return (n + 15) & ~(size_t)15; }

// Hidden columns per workgroup slice (the combine's outputs, and the out_proj
// front's x): H over the workgroups, rounded up to an even count, so that x
// travels in bf16 pairs that never straddle two slices.
static int slice_width(int H, int G) { return ((H + G - 1) / G + 1) & ~1; }

static LdsPlan lds_plan(const moe_tail_config* c, int G, int TC, size_t static_bytes, size_t limit) {
  LdsPlan L;
  const size_t R = c->max_rows, P = (size_t)c->max_rows * c->top_k, HR = (size_t)slice_width(c->hidden, G);
  L.xs = c->hidden + mt::XPAD;
  L.cs = TC * 32 + mt::XPAD;
  L.as = c->inter + mt::XPAD;
  L.ss = c->shared_inter + mt::XPAD;
  L.off_as = (int)al16((P + 1) * L.as * 2);
  L.off_outp = (int)(L.off_as + al16((R + 1) * L.ss * 2));
  L.off_shp = (int)(L.off_outp + al16(P * HR * 4));
  L.down = L.off_shp + al16((size_t)mt::NW * R * HR * 4);
  L.xn = (R + 1) * (size_t)L.xs * 2;
  L.chunk = (R + 1) * (size_t)L.cs * 2;
  // the out_proj front stages a K chunk of the attention rows first
  const size_t fr = c->attn_dim > 0 ? R * (size_t)mt::FRONT_AC * 2 : 0;
  size_t base = L.down > L.chunk ? L.down : L.chunk;
  base = base > fr ? base : fr;
  L.xn_lds = static_bytes + (L.xn > base ? L.xn : base) <= limit;
  L.dyn = L.xn_lds && L.xn > base ? L.xn : base;
  L.pa = (int)P;
  return L;
}

// The plan of a wide launch (R rows, 17..MAX_RW): xn stays in global scratch,
// and the down phase stages as many routed a rows at a time as fit (at least
// one slot's 16).  False if even that does not fit.
static bool lds_plan_wide(const moe_tail_config* c, int R, int G, int TC, size_t static_bytes, size_t limit,
                          LdsPlan* out) {
  LdsPlan L;
  const size_t P = (size_t)R * c->top_k, HR = (size_t)slice_width(c->hidden, G);
  L.xn_lds = 0;
  L.xs = c->hidden + mt::XPAD;
  L.cs = TC * 32 + mt::XPAD;
  L.as = c->inter + mt::XPAD;
  L.ss = c->shared_inter + mt::XPAD;
  L.xn = 0;
  L.chunk = (R + 1) * (size_t)L.cs * 2;
  // the routed a [pa + 1][as] and the shared a [R + 1][ss] share the first
  // region: the shared down is done before the routed a is staged
  const size_t fixed = al16(P * HR * 4) + al16((size_t)mt::NW * R * HR * 4);
  const size_t sa = al16((R + 1) * (size_t)L.ss * 2);
  if (static_bytes + fixed + sa > limit) return false;
  const size_t avail = limit - static_bytes - fixed;
  size_t pa = avail / ((size_t)L.as * 2);
  pa = pa > 0 ? pa - 1 : 0;
  if (pa > P) pa = P;
  while (pa >= 16 && al16((pa + 1) * (size_t)L.as * 2) > avail) --pa;
  if (pa < 16) return false;
  L.pa = (int)pa;
  const size_t ra = al16((pa + 1) * (size_t)L.as * 2);
  L.off_as = 0;
  L.off_outp = (int)(ra > sa ? ra : sa);
  L.off_shp = (int)(L.off_outp + al16(P * HR * 4));
  L.down = L.off_shp + al16((size_t)mt::NW * R * HR * 4);
  L.dyn = L.down > L.chunk ? L.down : L.chunk;
  if (static_bytes + L.dyn > limit) return false;
  *out = L;
  return true;
}

// K chunks per router/shared block: the smallest power of two (<= 16, dividing
// the workgroup count and H/32) that gives every workgroup a router chunk.
static int chunks_per_block(int H, int E, int G) {
  const int T1 = H / 32, n_rb = (E + 15) / 16;
  int S1 = 1;
  while (S1 < mt::NQ && n_rb * S1 < G && T1 % (2 * S1) == 0 && G % (2 * S1) == 0) S1 *= 2;
  return S1;
}

struct moe_tail {
  moe_tail_config cfg;
  int device;
  int G;
  size_t lds_dyn;
  LdsPlan plan;
  unsigned long long deadline_ticks;
  void* scratch;
  mt::Ctl* ctl;
  uint16_t* xn;
  uint64_t* xnt;
  uint64_t* lgt;
  uint64_t* part1;
  uint64_t* gpart;
  uint64_t* rstdt;
  size_t scratch_bytes;
  uint16_t* a_s;
  uint16_t* a_r;
  int S1, TC, n_rb, n_sb, Ep;
  int stall_spent;  // MOE_TAIL_DEBUG_STALL_ONCE: the first call has been launched
  int sticky;       // 1: an unread timeout makes later calls give up at once (handles); 0: each call starts clean
  int max_rows_call;  // the caller's max_rows (cfg.max_rows is a narrow launch's, at most MAX_R)
  int wide;           // calls of more than MAX_R rows run as one wide launch (else as narrow launches)
  int wide_only;      // the narrow plan does not fit: every call is a wide launch
  LdsPlan wplan;      // the wide launch's LDS plan
  size_t wlds_dyn;
  uint64_t* xft;      // [max_rows, H/2] tagged x pairs of the out_proj front (attn_dim > 0)
  char err[256];
};

static char g_create_err[256] = "";

static moe_tail_status fail(moe_tail_t* h, moe_tail_status st, const char* fmt, ...) {
  char* dst = h ? h->err : g_create_err;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(dst, 256, fmt, ap);
  va_end(ap);
  return st;
}

extern "C" moe_tail_status moe_tail_check_config(const moe_tail_config* c) {
  if (!c) return fail(nullptr, MOE_TAIL_EINVAL, "config is NULL");
  if (c->max_rows < 1 || c->max_rows > mt::MAX_ROWS_CALL)
    return fail(nullptr, MOE_TAIL_EINVAL, "max_rows %d outside 1..%d", c->max_rows, mt::MAX_ROWS_CALL);
  if (c->hidden < 128 || c->hidden > 16384 || c->hidden % 128)
    return fail(nullptr, MOE_TAIL_EINVAL, "hidden %d must be a multiple of 128 in 128..16384", c->hidden);
  if (c->num_experts < 1 || c->num_experts > mt::MAX_E)
    return fail(nullptr, MOE_TAIL_EINVAL, "num_experts %d outside 1..%d", c->num_experts, mt::MAX_E);
  if (c->top_k < 1 || c->top_k > mt::MAX_K || c->top_k > c->num_experts)
    return fail(nullptr, MOE_TAIL_EINVAL, "top_k %d outside 1..min(num_experts, %d)", c->top_k, mt::MAX_K);
  if (c->inter < 32 || c->inter > 4096 || c->inter % 32)
    return fail(nullptr, MOE_TAIL_EINVAL, "inter %d must be a multiple of 32 in 32..4096", c->inter);
  if (c->shared_inter < 0 || c->shared_inter > 4096 || c->shared_inter % 32)
    return fail(nullptr, MOE_TAIL_EINVAL, "shared_inter %d must be 0 or a multiple of 32 up to 4096", c->shared_inter);
  if (c->scoring != MOE_TAIL_SOFTMAX && c->scoring != MOE_TAIL_SIGMOID_BIAS)
    return fail(nullptr, MOE_TAIL_EINVAL, "unknown scoring %d", c->scoring);
  if (!(c->eps > 0.f) || !isfinite(c->eps)) return fail(nullptr, MOE_TAIL_EINVAL, "eps must be positive and finite");
  if (c->n_group < 0 || (c->n_group > 1 && (c->num_experts % c->n_group || (c->num_experts / c->n_group) % 8)))
    return fail(nullptr, MOE_TAIL_EINVAL, "n_group %d must divide num_experts %d into groups of a multiple of 8",
                c->n_group, c->num_experts);
  if (c->n_group > 1 && (c->topk_group < 1 || c->topk_group > c->n_group ||
                         c->top_k > c->topk_group * (c->num_experts / c->n_group)))
    return fail(nullptr, MOE_TAIL_EINVAL, "topk_group %d must be in 1..n_group and keep at least top_k experts",
                c->topk_group);
  if (c->attn_dim < 0 || c->attn_dim > 16384 || c->attn_dim % 128)
    return fail(nullptr, MOE_TAIL_EINVAL, "attn_dim %d must be 0 or a multiple of 128 up to 16384", c->attn_dim);
  if (c->w13_layout != 0 && !(c->w13_layout == 1 && c->weight_format == MOE_TAIL_MXFP4))
    return fail(nullptr, MOE_TAIL_EINVAL, "w13_layout %d: 0, or 1 with MXFP4 experts", c->w13_layout);
  if (c->fold_norm != 0 && c->fold_norm != 1)
    return fail(nullptr, MOE_TAIL_EINVAL, "fold_norm %d must be 0 or 1", c->fold_norm);
  if (c->weight_format != MOE_TAIL_MXFP4 && c->weight_format != MOE_TAIL_MXFP8)
    return fail(nullptr, MOE_TAIL_EINVAL, "unknown weight_format %d", c->weight_format);
  if (!(c->routed_scale >= 0.f) || !isfinite(c->routed_scale))
    return fail(nullptr, MOE_TAIL_EINVAL, "routed_scale must be finite and not negative");
  if (c->debug_flags & ~(MOE_TAIL_DEBUG_STALL | MOE_TAIL_DEBUG_STALL_ONCE))
    return fail(nullptr, MOE_TAIL_EINVAL, "unknown debug_flags bits");
  return MOE_TAIL_OK;
}

#define HIPCHK(h, call)                                                                       \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess) return fail((h), MOE_TAIL_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// What a handle needs to know of its device.
struct DevInfo {
  int G;                 // compute units = workgroups per launch
  size_t lds_per_block;  // bytes of LDS a workgroup may use
  int wclk_khz;          // wall-clock (s_memrealtime) rate
};

static moe_tail_status dev_info(int dev, DevInfo* di) {
  hipDeviceProp_t prop;
  HIPCHK(nullptr, hipGetDeviceProperties(&prop, dev));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  di->G = prop.multiProcessorCount;
  if (di->G > mt::MAX_G) return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "%d compute units, at most %d supported", di->G, mt::MAX_G);
  di->lds_per_block = (size_t)prop.sharedMemPerBlock;
  int wclk_khz = 0;
  HIPCHK(nullptr, hipDeviceGetAttribute(&wclk_khz, hipDeviceAttributeWallClockRate, dev));
  di->wclk_khz = wclk_khz > 0 ? wclk_khz : 100000;
  return MOE_TAIL_OK;
}

// Byte offsets of the scratch regions (each 256-byte aligned).
struct ScratchLayout {
  size_t o_ctl, o_xn, o_xnt, o_lg, o_pt, o_gp, o_rs, o_as, o_ar, o_xf, total;
};

// Every kernel of the tail, in the order: xn staged in LDS (8), xn from global
// scratch (4), wide launches (4).
static const void* const k_all[16] = {
    (const void*)mt::moe_tail_kernel_lds,    (const void*)mt::moe_tail_kernel_lds_rs,
    (const void*)mt::moe_tail_kernel_lds_f,  (const void*)mt::moe_tail_kernel_lds_rs_f,
    (const void*)mt::moe_tail_kernel_lds_8,  (const void*)mt::moe_tail_kernel_lds_rs_8,
    (const void*)mt::moe_tail_kernel_lds_f8, (const void*)mt::moe_tail_kernel_lds_rs_f8,
    (const void*)mt::moe_tail_kernel_gm,     (const void*)mt::moe_tail_kernel_gm_f,
    (const void*)mt::moe_tail_kernel_gm_8,   (const void*)mt::moe_tail_kernel_gm_f8,
    (const void*)mt::moe_tail_kernel_gm_w,   (const void*)mt::moe_tail_kernel_gm_wf,
    (const void*)mt::moe_tail_kernel_gm_w8,  (const void*)mt::moe_tail_kernel_gm_wf8};

// Fill every field of h that depends only on the configuration and the device
// (no allocation, no pointer into scratch yet) and the scratch layout it needs.
static moe_tail_status plan_handle(const moe_tail_config* cfg_in, int dev, const DevInfo& di, moe_tail_t* h,
                                   ScratchLayout* L, bool allow_wide = true) {
  moe_tail_status st = moe_tail_check_config(cfg_in);
  if (st != MOE_TAIL_OK) return st;
  // everything below is sized per launch: at most MAX_R rows
  moe_tail_config icfg = *cfg_in;
  if (icfg.max_rows > mt::MAX_R) icfg.max_rows = mt::MAX_R;
  const moe_tail_config* cfg = &icfg;
  const int G = di.G;
  hipFuncAttributes fa;
  HIPCHK(nullptr, hipFuncGetAttributes(&fa, (const void*)mt::moe_tail_kernel_lds));
  const int S1 = chunks_per_block(cfg->hidden, cfg->num_experts, G), TC = cfg->hidden / 32 / S1;
  const int n_rb = (cfg->num_experts + 15) / 16, n_sb = cfg->shared_inter / 8;
  const int n_it = (n_rb + n_sb) * S1;
  if ((n_it + G - 1) / G > mt::MAX_ITEMS1)
    return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "%d router/shared items exceed %d per workgroup", n_it, mt::MAX_ITEMS1);
  const LdsPlan plan = lds_plan(cfg, G, TC, fa.sharedSizeBytes, di.lds_per_block);
  const bool narrow_fits = plan.dyn + fa.sharedSizeBytes <= di.lds_per_block;
  if (slice_width(cfg->hidden, G) > 16 * mt::MAX_BLK)
    return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "hidden %d too large for %d workgroups", cfg->hidden, G);
  // The wide launch: more than MAX_R rows in one launch, or every call where
  // the narrow plan does not fit (its routed a staged in groups), when its
  // own plan fits (not with the out_proj front, whose attention chunk is
  // staged for MAX_R rows)
  LdsPlan wplan;
  memset(&wplan, 0, sizeof(wplan));
  bool wide = false;
  if (allow_wide && (cfg_in->max_rows > mt::MAX_R || !narrow_fits) && cfg_in->attn_dim == 0 &&
      cfg_in->max_rows * cfg_in->top_k <= mt::MAX_P) {
    HIPCHK(nullptr, hipFuncGetAttributes(&fa, (const void*)mt::moe_tail_kernel_gm_w));
    wide = lds_plan_wide(cfg_in, cfg_in->max_rows, G, TC, fa.sharedSizeBytes, di.lds_per_block, &wplan);
  }
  if (!narrow_fits && !wide)
    return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "needs %zu B of LDS, device has %zu", plan.dyn + fa.sharedSizeBytes,
                di.lds_per_block);
  memset(h, 0, sizeof(*h));
  h->cfg = *cfg;
  h->max_rows_call = cfg_in->max_rows;
  h->wide = wide;
  h->wide_only = !narrow_fits;
  h->wplan = wplan;
  h->wlds_dyn = wide ? wplan.dyn : 0;
  h->device = dev;
  h->G = G;
  h->lds_dyn = plan.dyn;
  h->plan = plan;
  const unsigned long long us = cfg->deadline_us ? cfg->deadline_us : 200000u;
  h->deadline_ticks = us * (unsigned long long)di.wclk_khz / 1000ull;
  h->S1 = S1;
  h->TC = TC;
  h->n_rb = n_rb;
  h->n_sb = n_sb;
  h->Ep = (cfg->num_experts + 7) & ~7;
  h->sticky = 1;
  // rows of the widest launch; a wide launch's K-chunk partials have 32 columns
  const size_t R = wide ? cfg_in->max_rows : cfg->max_rows, H = cfg->hidden, K = cfg->top_k;
  const size_t I = cfg->inter, Is = cfg->shared_inter, PCOL = wide ? 32 : 16;
  auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
  L->o_ctl = 0;
  L->o_xn = L->o_ctl + al(sizeof(mt::Ctl));
  L->o_xnt = L->o_xn + al(R * H * 2);
  L->o_lg = L->o_xnt + al(R * H * 4);
  L->o_pt = L->o_lg + al(R * (size_t)h->Ep * 8);
  L->o_gp = L->o_pt + al((size_t)n_it * PCOL * 128);
  L->o_rs = L->o_gp + al(R * mt::NQ * 8);
  L->o_as = L->o_rs + al(R * 8);
  L->o_ar = L->o_as + al(R * (Is ? Is : 1) * 2);
  L->o_xf = L->o_ar + al(R * K * I * 2);
  L->total = L->o_xf + (cfg->attn_dim > 0 ? al(R * H * 4) : 0);
  snprintf(h->err, sizeof(h->err), "no error");
  return MOE_TAIL_OK;
}

// Point the handle's regions into scratch memory that starts at base.
static void place_scratch(moe_tail_t* h, const ScratchLayout& L, void* base_) {
  char* base = (char*)base_;
  h->scratch = base_;
  h->scratch_bytes = L.total;
  h->ctl = (mt::Ctl*)(base + L.o_ctl);
  h->xn = (uint16_t*)(base + L.o_xn);
  h->xnt = (uint64_t*)(base + L.o_xnt);
  h->lgt = (uint64_t*)(base + L.o_lg);
  h->part1 = (uint64_t*)(base + L.o_pt);
  h->gpart = (uint64_t*)(base + L.o_gp);
  h->rstdt = (uint64_t*)(base + L.o_rs);
  h->a_s = (uint16_t*)(base + L.o_as);
  h->a_r = (uint16_t*)(base + L.o_ar);
  h->xft = h->cfg.attn_dim > 0 ? (uint64_t*)(base + L.o_xf) : nullptr;
}

// Let every kernel use all the LDS a workgroup may have (a launch then asks
// for its own dynamic size; handles of different sizes never narrow each
// other's limit), and check that one workgroup of each kernel this handle
// may launch fits on a compute unit at the handle's dynamic LDS size: every
// cross-workgroup wait assumes that all G workgroups are resident at once
// (one per compute unit), which a plain launch relies on.  Call with the
// handle's device current.
static moe_tail_status prepare_kernels(const moe_tail_t* h, const DevInfo& di) {
  for (int k = 0; k < 16; ++k) {
    hipFuncAttributes fa;
    HIPCHK(nullptr, hipFuncGetAttributes(&fa, k_all[k]));
    const int lim = (int)(di.lds_per_block - fa.sharedSizeBytes);
    HIPCHK(nullptr, hipFuncSetAttribute(k_all[k], hipFuncAttributeMaxDynamicSharedMemorySize, lim));
  }
  const bool xl = h->plan.xn_lds;
  for (int k = h->wide_only ? 12 : xl ? 0 : 8; k < (h->wide ? 16 : xl ? 8 : 12); ++k) {
    if (xl && k >= 8 && k < 12) continue;
    const size_t dyn = k >= 12 ? h->wlds_dyn : h->lds_dyn;
    int nb = 0;
    HIPCHK(nullptr, hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_all[k], mt::NT, dyn));
    if (nb < 1)
      return fail(nullptr, MOE_TAIL_EUNSUPPORTED,
                  "a workgroup of %d threads with %zu B of dynamic LDS does not fit on a compute unit", mt::NT, dyn);
  }
  return MOE_TAIL_OK;
}

extern "C" moe_tail_status moe_tail_create(const moe_tail_config* cfg, moe_tail_t** out) {
  if (!out) return fail(nullptr, MOE_TAIL_EINVAL, "out is NULL");
  *out = nullptr;
  moe_tail_status st = moe_tail_check_config(cfg);
  if (st != MOE_TAIL_OK) return st;
  int dev = cfg->device;
  if (dev < 0) HIPCHK(nullptr, hipGetDevice(&dev));
  DevInfo di;
  if ((st = dev_info(dev, &di)) != MOE_TAIL_OK) return st;
  moe_tail_t* h = (moe_tail_t*)calloc(1, sizeof(moe_tail_t));
  if (!h) return fail(nullptr, MOE_TAIL_ENOMEM, "host allocation failed");
  ScratchLayout L;
  if ((st = plan_handle(cfg, dev, di, h, &L)) != MOE_TAIL_OK) {
    free(h);
    return st;
  }
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(dev);
  void* base = nullptr;
  hipError_t e = hipMalloc(&base, L.total);
  if (e != hipSuccess) {
    (void)hipSetDevice(prev);
    free(h);
    return fail(nullptr, MOE_TAIL_ENOMEM, "hipMalloc(%zu): %s", L.total, hipGetErrorString(e));
  }
  place_scratch(h, L, base);
  e = hipMemset(base, 0, L.total);
  if (e == hipSuccess) st = prepare_kernels(h, di);
  if (e == hipSuccess && st == MOE_TAIL_OK) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess || st != MOE_TAIL_OK) {
    (void)hipFree(base);
    free(h);
    return e != hipSuccess ? fail(nullptr, MOE_TAIL_EHIP, "scratch setup: %s", hipGetErrorString(e)) : st;
  }
  *out = h;
  return MOE_TAIL_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// One launch: narrow over rows <= MAX_R, or wide over more (handles with wide set).
static moe_tail_status run_launch(moe_tail_t* h, int32_t rows, const moe_tail_args* a, void* stream) {
  const moe_tail_config& c = h->cfg;
  const bool wide = h->wide && (rows > c.max_rows || h->wide_only);
  const int lim = wide ? h->max_rows_call : c.max_rows;
  if (rows < 1 || rows > lim) return fail(h, MOE_TAIL_EINVAL, "rows %d outside 1..%d", rows, lim);
  const LdsPlan& pl = wide ? h->wplan : h->plan;
  // x, or attention rows for the out_proj front (checked by the caller)
  const void* req[] = {a->attn ? a->attn : a->x, a->gamma, a->router_w, a->w13_q, a->w13_s, a->w2_q, a->w2_s, a->out};
  const char* names[] = {"x", "gamma", "router_w", "w13_q", "w13_s", "w2_q", "w2_s", "out"};
  for (int k = 0; k < 8; ++k) {
    if (!req[k]) return fail(h, MOE_TAIL_EINVAL, "%s is NULL", names[k]);
    if (!aligned(req[k], 16)) return fail(h, MOE_TAIL_EINVAL, "%s is not 16-byte aligned", names[k]);
  }
  if (a->residual && !aligned(a->residual, 16)) return fail(h, MOE_TAIL_EINVAL, "residual is not 16-byte aligned");
  if (a->res_out && !aligned(a->res_out, 16)) return fail(h, MOE_TAIL_EINVAL, "res_out is not 16-byte aligned");
  if (a->shared_gate && !aligned(a->shared_gate, 16))
    return fail(h, MOE_TAIL_EINVAL, "shared_gate is not 16-byte aligned");
  if (c.scoring == MOE_TAIL_SIGMOID_BIAS && (!a->router_bias || !aligned(a->router_bias, 4)))
    return fail(h, MOE_TAIL_EINVAL, "router_bias is required (4-byte aligned) for sigmoid scoring");
  if (c.shared_inter > 0) {
    if (!a->ws13 || !a->ws2) return fail(h, MOE_TAIL_EINVAL, "ws13 and ws2 are required when shared_inter > 0");
    if (!aligned(a->ws13, 16) || !aligned(a->ws2, 16))
      return fail(h, MOE_TAIL_EINVAL, "ws13/ws2 are not 16-byte aligned");
  }
  const void* o4[] = {a->topk_ids, a->topk_w, a->dbg_logits, a->dbg_y_routed, a->dbg_y_shared};
  for (int k = 0; k < 5; ++k)
    if (o4[k] && !aligned(o4[k], 4)) return fail(h, MOE_TAIL_EINVAL, "an fp32/int32 output is not 4-byte aligned");

  mt::Params p;
  p.R = rows;
  p.H = c.hidden;
  p.E = c.num_experts;
  p.K = c.top_k;
  p.I = c.inter;
  p.Is = c.shared_inter;
  p.scoring = c.scoring;
  p.n_group = c.n_group > 1 ? c.n_group : 1;
  p.topk_group = c.n_group > 1 ? c.topk_group : 1;
  p.rscale = c.routed_scale > 0.f ? c.routed_scale : 1.f;
  p.f8 = c.weight_format == MOE_TAIL_MXFP8;
  p.fold = c.fold_norm;
  p.shuf = c.w13_layout == 1;
  p.G = h->G;
  p.xn_lds = pl.xn_lds;
  // reader-side router sums when each thread then loads at most 8 partials
  p.rsum = p.xn_lds && rows * c.num_experts * h->S1 <= 8192 && rows * c.num_experts <= mt::RED_FLOATS;
  p.xs = pl.xs;
  p.cs = pl.cs;
  p.n_rb = h->n_rb;
  p.n_sb = h->n_sb;
  {  // the norm's workgroups take no router/shared items when they are few
     // (up to 2 rows: measured faster at 1 and 2 rows; at 4 rows it depends
     // on the shape, slower at c1's and faster at c3's, so it stays off)
    const int nn = rows * mt::NQ;
    p.nn1 = nn <= 2 * mt::NQ && nn % h->S1 == 0 && h->G - nn >= h->S1 &&
                    ((h->n_rb + h->n_sb) * h->S1 + (h->G - nn) - 1) / (h->G - nn) <= mt::MAX_ITEMS1
                ? nn
                : 0;
  }
  p.S1 = h->S1;
  p.TC = h->TC;
  p.Ep = h->Ep;
  p.as = pl.as;
  p.ss = pl.ss;
  p.off_as = pl.off_as;
  p.off_outp = pl.off_outp;
  p.off_shp = pl.off_shp;
  p.xzero = wide ? h->max_rows_call : c.max_rows;
  p.azero = wide ? pl.pa : c.max_rows * c.top_k;
  p.szero = p.xzero;
  p.eps = (double)c.eps;
  p.deadline_ticks = h->deadline_ticks;
  p.debug_flags = c.debug_flags & MOE_TAIL_DEBUG_STALL;
  if ((c.debug_flags & MOE_TAIL_DEBUG_STALL_ONCE) && !h->stall_spent) {
    p.debug_flags |= MOE_TAIL_DEBUG_STALL;
    h->stall_spent = 1;
  }
  p.debug_block = c.debug_block;
  p.sticky = h->sticky;
  p.x = (const uint16_t*)a->x;
  p.res = (const uint16_t*)a->residual;
  p.gamma = (const uint16_t*)a->gamma;
  p.rw = (const uint16_t*)a->router_w;
  p.bias = a->router_bias;
  p.w13q = a->w13_q;
  p.w13s = a->w13_s;
  p.w2q = a->w2_q;
  p.w2s = a->w2_s;
  p.ws13 = (const uint16_t*)a->ws13;
  p.ws2 = (const uint16_t*)a->ws2;
  p.sgate = (const uint16_t*)a->shared_gate;
  p.attn = (const uint16_t*)a->attn;
  p.w_o = a->attn ? (const uint16_t*)a->w_o : nullptr;
  p.A = a->attn ? c.attn_dim : 0;
  p.HR = slice_width(c.hidden, h->G);
  p.xft = h->xft;
  p.out = (uint16_t*)a->out;
  p.res_out = (uint16_t*)a->res_out;
  p.topk_ids = a->topk_ids;
  p.topk_w = a->topk_w;
  p.dbg_logits = a->dbg_logits;
  p.dbg_yr = a->dbg_y_routed;
  p.dbg_ys = a->dbg_y_shared;
  p.ctl = h->ctl;
  p.xn = h->xn;
  p.xnt = h->xnt;
  p.lgt = h->lgt;
  p.part1 = h->part1;
  p.gpart = h->gpart;
  p.rstdt = h->rstdt;
  p.a_s = h->a_s;
  p.a_r = h->a_r;

  // A plain launch, eager or captured alike: create() has checked that one
  // workgroup fits on every compute unit, so all G are resident together on
  // an otherwise idle device; a wait that is never met (another kernel holding
  // compute units) ends at its deadline with ETIMEOUT instead of hanging.
  void* kargs[] = {&p};
  const void* kern = mt::kernel_for(p, wide);
  const hipError_t e =
      hipLaunchKernel(kern, dim3(h->G), dim3(mt::NT), kargs, wide ? h->wlds_dyn : h->lds_dyn, (hipStream_t)stream);
  if (e != hipSuccess) return fail(h, MOE_TAIL_EHIP, "kernel launch: %s", hipGetErrorString(e));
  return MOE_TAIL_OK;
}

extern "C" moe_tail_status moe_tail_run(moe_tail_t* h, int32_t rows, const moe_tail_args* a, void* stream) {
  if (!h) return fail(nullptr, MOE_TAIL_EINVAL, "handle is NULL");
  if (!a) return fail(h, MOE_TAIL_EINVAL, "args is NULL");
  if (rows < 1 || rows > h->max_rows_call)
    return fail(h, MOE_TAIL_EINVAL, "rows %d outside 1..%d", rows, h->max_rows_call);
  if (a->attn) {  // the out_proj front: x = bf16(attn . w_o^T), computed in the same launch as the tail
    if (a->x) return fail(h, MOE_TAIL_EINVAL, "give x or attn, not both");
    if (!h->xft) return fail(h, MOE_TAIL_EINVAL, "attn needs a handle created with attn_dim > 0");
    if (!a->w_o) return fail(h, MOE_TAIL_EINVAL, "w_o is required with attn");
    if (!aligned(a->attn, 16) || !aligned(a->w_o, 16)) return fail(h, MOE_TAIL_EINVAL, "attn/w_o are not 16-byte aligned");
    if (h->cfg.fold_norm) return fail(h, MOE_TAIL_EUNSUPPORTED, "the folded norm does not take attn (it reads x by chunks)");
  }
  if (rows <= mt::MAX_R || h->wide) return run_launch(h, rows, a, stream);
  // More rows than a narrow launch's MFMA columns, on a handle without the
  // wide launch: balanced row ranges, one launch each, in order on the
  // stream (each streams its own experts)
  const int n = (rows + mt::MAX_R - 1) / mt::MAX_R;
  const size_t H = h->cfg.hidden, E = h->cfg.num_experts, K = h->cfg.top_k;
  for (int i = 0; i < n; ++i) {
    const int r0 = i * rows / n, r1 = (i + 1) * rows / n;
    moe_tail_args b = *a;
    auto off16 = [&](const void* q, size_t per_row) -> void* {
      return q ? (void*)((const uint16_t*)q + (size_t)r0 * per_row) : nullptr;
    };
    auto off32 = [&](const void* q, size_t per_row) -> void* {
      return q ? (void*)((const uint32_t*)q + (size_t)r0 * per_row) : nullptr;
    };
    b.x = off16(a->x, H);
    b.attn = off16(a->attn, (size_t)h->cfg.attn_dim);
    b.residual = off16(a->residual, H);
    b.out = (uint16_t*)off16(a->out, H);
    b.res_out = (uint16_t*)off16(a->res_out, H);
    b.topk_ids = (int32_t*)off32(a->topk_ids, K);
    b.topk_w = (float*)off32(a->topk_w, K);
    b.dbg_logits = (float*)off32(a->dbg_logits, E);
    b.dbg_y_routed = (float*)off32(a->dbg_y_routed, H);
    b.dbg_y_shared = (float*)off32(a->dbg_y_shared, H);
    const moe_tail_status st = run_launch(h, r1 - r0, &b, stream);
    if (st != MOE_TAIL_OK) return st;
  }
  return MOE_TAIL_OK;
}

extern "C" moe_tail_status moe_tail_get_error(moe_tail_t* h) {
  if (!h) return fail(nullptr, MOE_TAIL_EINVAL, "handle is NULL");
  uint32_t w[8] = {0};
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(w, &h->ctl->error, sizeof(w), hipMemcpyDeviceToHost);
  const uint32_t v = w[0];
  uint32_t ep_lo = 0, ep_hi = 0;
  if (e == hipSuccess && v) {  // the workgroups' epochs, for the message
    static_assert(sizeof(mt::Ctl::cta_ep[0]) == 64, "one line per workgroup");
    std::vector<uint32_t> eps((size_t)h->G * 16);
    e = hipMemcpy(eps.data(), h->ctl->cta_ep, eps.size() * 4, hipMemcpyDeviceToHost);
    ep_lo = ep_hi = eps[0];
    for (int i = 1; i < h->G; ++i) {
      ep_lo = eps[i * 16] < ep_lo ? eps[i * 16] : ep_lo;
      ep_hi = eps[i * 16] > ep_hi ? eps[i * 16] : ep_hi;
    }
  }
  // after a failed call the workgroups' epochs and counters may disagree:
  // start the handle's scratch over (nothing is in flight now).  The epochs
  // restart, so the tagged words are cleared with them.
  if (e == hipSuccess && v) e = hipMemset(h->scratch, 0, h->scratch_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail(h, MOE_TAIL_EHIP, "reading the error word: %s", hipGetErrorString(e));
  static const char* names[4] = {"norm", "router", "shared", "routed"};
  if (v == MOE_TAIL_ETIMEOUT)
    return fail(h, MOE_TAIL_ETIMEOUT,
                "a cross-workgroup wait passed its deadline: %s wait in workgroup %u saw %u of %u (epoch %u, info %u; "
                "workgroup epochs now %u..%u)",
                w[1] < 4 ? names[w[1]] : "?", w[2], w[3], w[4], w[5], w[6], ep_lo, ep_hi);
  return MOE_TAIL_OK;
}

// ------------------------------------------------ the no-allocation entry --

// Scratch of moe_tail_run_noalloc: one array per device, zero when the code
// object loads, kept for the life of the process.  Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in for
// the symbol): it uses the device address that hipGetSymbolAddress returns
// for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_TAIL_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEV = 64;
struct NoallocDev {
  int ready;         // ptr and info are valid
  void* ptr;         // this device's address of `scratch`
  DevInfo info;
  size_t lds_ready;  // largest dynamic LDS size prepared so far, per kernel family (0: none)
  size_t lds_ready_gm;
  size_t lds_ready_w;
};
NoallocDev g_noalloc[NOALLOC_MAX_DEV];
std::mutex g_noalloc_mu;
}  // namespace

extern "C" moe_tail_status moe_tail_run_noalloc(const moe_tail_config* cfg, int32_t rows, const moe_tail_args* a,
                                                void* stream) {
  moe_tail_status st = moe_tail_check_config(cfg);
  if (st != MOE_TAIL_OK) return st;
  if (cfg->debug_flags & MOE_TAIL_DEBUG_STALL_ONCE)
    return fail(nullptr, MOE_TAIL_EINVAL, "MOE_TAIL_DEBUG_STALL_ONCE needs a handle");
  int dev = 0;
  HIPCHK(nullptr, hipGetDevice(&dev));
  if (cfg->device >= 0 && cfg->device != dev)
    return fail(nullptr, MOE_TAIL_EINVAL, "config device %d is not the current device %d", cfg->device, dev);
  if (dev >= NOALLOC_MAX_DEV) return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "device %d beyond %d", dev, NOALLOC_MAX_DEV);
  moe_tail_t h;  // a handle on the stack over the static scratch; nothing is allocated
  ScratchLayout L;
  {
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    NoallocDev& d = g_noalloc[dev];
    if (!d.ready) {  // once per device, with that device current
      void* ptr = nullptr;
      HIPCHK(nullptr, hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
      if ((st = dev_info(dev, &d.info)) != MOE_TAIL_OK) return st;
      d.ptr = ptr;
      d.ready = 1;
    }
    if ((st = plan_handle(cfg, dev, d.info, &h, &L)) != MOE_TAIL_OK) return st;
    // a wide launch's scratch (32-column partials, all rows) may not fit where
    // narrow launches' does: then calls above 16 rows run as narrow launches
    if (L.total > sizeof(scratch) && h.wide && (st = plan_handle(cfg, dev, d.info, &h, &L, false)) != MOE_TAIL_OK)
      return st;
    if (L.total > sizeof(scratch))
      return fail(nullptr, MOE_TAIL_EINVAL, "this configuration needs %zu B of scratch; moe_tail_run_noalloc has %zu",
                  L.total, sizeof(scratch));
    // the residency check passed at this dynamic LDS size or a larger one
    size_t& done = h.plan.xn_lds ? d.lds_ready : d.lds_ready_gm;
    const bool need_n = !h.wide_only && (h.lds_dyn > done || !done);
    const bool need_w = h.wide && (h.wlds_dyn > d.lds_ready_w || !d.lds_ready_w);
    if (need_n || need_w) {
      if ((st = prepare_kernels(&h, d.info)) != MOE_TAIL_OK) return st;
      if (!h.wide_only && h.lds_dyn > done) done = h.lds_dyn;
      if (h.wide && h.wlds_dyn > d.lds_ready_w) d.lds_ready_w = h.wlds_dyn;
    }
    place_scratch(&h, L, d.ptr);
  }
  h.sticky = 0;  // nothing reads this scratch's error word: each call starts clean
  st = moe_tail_run(&h, rows, a, stream);
  if (st != MOE_TAIL_OK) snprintf(g_create_err, sizeof(g_create_err), "%s", h.err);
  return st;
}

#ifdef MOE_TAIL_TIMELINE
// Timeline builds only: copy the last call's stamps ([1024][16] u64) to host.
extern "C" int moe_tail_debug_timeline(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(mt::g_timeline), sizeof(mt::g_timeline), 0,
                                  hipMemcpyDeviceToHost);
}
#endif

extern "C" const char* moe_tail_strerror(moe_tail_t* h) { return h ? h->err : g_create_err; }

extern "C" void moe_tail_destroy(moe_tail_t* h) {
  if (!h) return;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->device);
  (void)hipFree(h->scratch);
  (void)hipSetDevice(prev);
  free(h);
}
