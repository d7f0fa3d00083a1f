// Device code of the fused decode MoE layer tail (gfx950): the kernel body,
// shared by the narrow kernels (moe_tail.hip) and the wide ones
// (moe_tail_wide.hip).  The steps and their sources are described at the
// top of moe_tail.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "moe_tail.h"

namespace mt {

constexpr int NT = 512;      // threads per workgroup
constexpr int NW = NT / 64;  // waves per workgroup
constexpr int NQ = 16;       // norm slices per row
constexpr int MAX_R = 16;          // rows per narrow launch (one tile of MFMA columns)
constexpr int MAX_RW = 32;         // rows per wide launch (two tiles of MFMA columns)
constexpr int MAX_ROWS_CALL = 32;  // rows per call
constexpr int MAX_E = 512;
constexpr int MAX_K = 32;
constexpr int MAX_P = MAX_R * MAX_K;  // picks per launch (a wide launch needs rows x top_k <= MAX_P)
constexpr int MAX_BLK = 2;            // 16-row down blocks per workgroup
constexpr int D_BF = 12;              // bf16 weight loads in flight per wave
constexpr int D_FP4_G = 4;            // MXFP4 items in flight per wave when activations come from global memory
constexpr int XPAD = 8;               // bf16 padding per LDS activation row
constexpr int FRONT_AC = 1024;                       // out_proj front: attention columns per K chunk
constexpr int FRONT_WV = FRONT_AC / 8 / 16;          // its weight vectors per thread and chunk
constexpr int FRONT_AV = MAX_R * FRONT_AC / 8 / NT;  // its attention vectors per thread and chunk (staged in LDS; narrow launches only)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MAX_U1 = 32 + 512;  // router blocks (E/16) + shared blocks (Is/8)
constexpr int MAX_G = 1024;        // workgroups (one per compute unit)
constexpr int NRC = 16;            // routed-arrival counters (workgroup c adds to c % NRC)
constexpr int MAX_ITEMS1 = 64;     // K-chunk items of the router/shared phase per workgroup

// Arrival counters of one call.  Every counter sits on its own 64-byte line;
// contention on one address serialises the atomics, so each counter has a
// small fan-in (at most 16 arrivals, 512 for the shared blocks, whose wait is
// off the critical path).  The router's results need no counter: they travel
// as tagged words.
struct Bank {
  uint32_t normc[NQ][16];     // norm slice q: one arrival per row
  uint32_t shared[16];        // shared blocks whose activations are final
  uint32_t routed[NRC][16];   // routed gate/up units done
  uint32_t abort_[16];        // set by a wait that passed its deadline
  uint32_t unitc[MAX_U1][16]; // K-chunk partials stored, per router/shared block
};
constexpr int BANK_WORDS = (int)(sizeof(Bank) / 4);

struct Ctl {
  uint32_t error;
  uint32_t diag[7];  // first timeout: wait id, workgroup, observed, target, epoch, info
  uint32_t _p0[56];
  uint32_t cta_ep[MAX_G][16];  // per workgroup, one line each: calls it has started (its epoch)
  Bank bank[2];
};

struct Params {
  int R, H, E, K, I, Is, scoring, G;
  int n_group, topk_group;  // group-limited routing (n_group 1: none)
  int f8;                   // routed experts in MXFP8 (E4M3 codes), else MXFP4
  int fold;                 // rstd multiplies the router and shared gate/up sums over bf16(h * gamma)
  int shuf;                 // MXFP4 w13 codes in the unit-blocked layout (one 1 KB block per wave load)
  float rscale;             // routed scaling factor
  int xn_lds;                     // activations staged in LDS (else read from global scratch)
  int rsum;                       // top-k readers sum the router K-chunk partials themselves
  int xs, as, ss;                 // LDS row strides (bf16 elements): xn, routed a, shared a
  int cs;                         // LDS row stride of the router/shared phase's xn chunk
  int off_as, off_outp, off_shp;  // byte offsets in dynamic LDS (down phase)
  int xzero, azero, szero;        // indices of the all-zero LDS rows (inactive MFMA columns); a wide
                                  // launch stages up to azero routed a rows at a time
  int n_rb, n_sb;                 // router blocks (16 experts), shared blocks (8 gate + 8 up rows)
  int nn1;                        // leading workgroups that take no router/shared items (the norm's, at few rows)
  int S1, TC;                     // K chunks per block, 32-column groups per chunk
  int Ep;                         // logits row stride (E rounded up to 8)
  double eps;
  unsigned long long deadline_ticks;
  uint32_t debug_flags;
  int debug_block;
  int sticky;  // an unread earlier timeout makes this call give up at its first unmet wait
  const uint16_t* x;
  const uint16_t* res;
  const uint16_t* gamma;
  const uint16_t* rw;
  const float* bias;
  const uint8_t* w13q;
  const uint8_t* w13s;
  const uint8_t* w2q;
  const uint8_t* w2s;
  const uint16_t* ws13;
  const uint16_t* ws2;
  const uint16_t* sgate;  // [H] shared-expert gate, or null
  const uint16_t* attn;   // [R][A] attention rows in place of x (the out_proj front), or null
  const uint16_t* w_o;    // [H][A] out_proj weights (with attn)
  int A;                  // attention width
  int HR;                 // hidden columns per workgroup slice (even)
  uint16_t* out;
  uint16_t* res_out;
  int32_t* topk_ids;
  float* topk_w;
  float* dbg_logits;
  float* dbg_yr;
  float* dbg_ys;
  Ctl* ctl;
  uint16_t* xn;
  uint64_t* xnt;    // [R][H/2] tagged xn pairs (this call's K-chunk readers)
  uint64_t* lgt;    // [R][Ep] tagged fp32 logits
  uint64_t* part1;  // [blocks * S1][16 or, wide, 32 rows][16] tagged fp32 K-chunk partial sums
  uint64_t* gpart;  // [R][NQ] tagged fp32 partial dots of the shared gate, one per norm slice
  uint64_t* rstdt;  // [R] tagged fp32 rstd of each row (folded norm)
  uint64_t* xft;    // [R][H/2] tagged x pairs computed by the out_proj front, one slice per workgroup
  uint16_t* a_s;
  uint16_t* a_r;
};

// ------------------------------------------------------------------ helpers --

// Buffer accesses.  Weights use the default cache policy: an MFMA operand
// load covers 64 bytes of each of 16 rows, so a 128-byte line is consumed by
// two consecutive loads (and a line of block scales by eight), and a
// nontemporal policy, which does not keep the line for the next load,
// measured slower on MI355X (5.5 vs 6.3 TB/s for this pattern).
// Out-of-range offsets read 0 without touching memory, which pads ragged
// tiles and the tails of the load windows.  Exchanged scratch (xn, logits,
// a) is written and read with device-scope (SC1) accesses, coherent across
// the XCDs' L2s, so no L2 write-back or invalidate is ever needed.
constexpr int CP_W = 0;
constexpr int CP_SC1 = 16;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// The same for a base and size that are uniform but that the compiler may keep
// in vector registers: read from the first lane, so the load needs no
// per-lane descriptor loop.
__device__ __forceinline__ rsrc_t make_rsrc_u(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t nb = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
  return make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo), nb);
}
template <int CP>
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP));
}
template <int CP>
__device__ __forceinline__ uint32_t ld4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, CP);
}
__device__ __forceinline__ void stc16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v),
                                         r, (int)off, 0, CP_SC1);
}
__device__ __forceinline__ void stc2(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, CP_SC1);
}
__device__ __forceinline__ u32x4 lds16(const void* p) { return *(const u32x4*)p; }

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16, nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// double -> bf16, nearest even, rounded once: round to odd at float precision
// (24 bits >= 8 + 2), then nearest even to bf16.
__device__ __forceinline__ uint32_t d2bf(double d) {
  float t = __double2float_rz(d);
  uint32_t u = __float_as_uint(t);
  if ((double)t != d) u |= 1u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E8M0 scale byte -> float 2^(s-127)
__device__ __forceinline__ float e8m0f(uint32_t s) { return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u); }

// 8 FP4 codes (one dword, element 0 in the low nibble) -> 8 bf16 times scale
__device__ __forceinline__ bf16x8 fp4x8(uint32_t v, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
  return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 E4M3 codes (two dwords, element 0 in the low byte) -> 8 bf16 times scale
// (E4M3 x 2^(s-127) is exact in bf16 for the scales in range)
__device__ __forceinline__ bf16x8 fp8x8(uint32_t lo, uint32_t hi, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// monotone map of a float onto uint32 (larger float -> larger key); -0 == +0;
// every finite key maps above 0, which marks a removed or absent expert
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// the float a key came from (finite floats only)
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide reductions to lane 63 with DPP row shifts and row broadcasts,
// read back as a uniform value.  Lanes without a DPP source take the identity.
template <int CTRL, int RMASK>
__device__ __forceinline__ int dpp(int id, int v) {
  return __builtin_amdgcn_update_dpp(id, v, CTRL, RMASK, 0xF, false);
}
#define WAVE_REDUCE(v, OP, ID)                 \
  v = OP(v, dpp<0x111, 0xF>((ID), (v)));       \
  v = OP(v, dpp<0x112, 0xF>((ID), (v)));       \
  v = OP(v, dpp<0x114, 0xF>((ID), (v)));       \
  v = OP(v, dpp<0x118, 0xF>((ID), (v)));       \
  v = OP(v, dpp<0x142, 0xA>((ID), (v)));       \
  v = OP(v, dpp<0x143, 0xC>((ID), (v)));
__device__ __forceinline__ int umax_(int a, int b) { return (uint32_t)a > (uint32_t)b ? a : b; }
__device__ __forceinline__ int fadd_(int a, int b) { return __float_as_int(__int_as_float(a) + __int_as_float(b)); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  int v = (int)x;
  WAVE_REDUCE(v, umax_, 0)
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  int v = __float_as_int(x);
  WAVE_REDUCE(v, fadd_, 0)
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}
template <int CTRL, int RMASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = dpp<CTRL, RMASK>(0, __double2loint(v));
  const int hi = dpp<CTRL, RMASK>(0, __double2hiint(v));
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0x111, 0xF>(v);
  v += dpp_f64<0x112, 0xF>(v);
  v += dpp_f64<0x114, 0xF>(v);
  v += dpp_f64<0x118, 0xF>(v);
  v += dpp_f64<0x142, 0xA>(v);
  v += dpp_f64<0x143, 0xC>(v);
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                          __builtin_amdgcn_readlane(__double2loint(v), 63));
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int l = threadIdx.x & 63;
  return l ? (~0ull >> (64 - l)) : 0ull;
}

// index of the n-th set bit of m (n < popcount(m))
__device__ __forceinline__ int nth_bit(uint32_t m, int n) {
  for (int k = 0; k < n; ++k) m &= m - 1;
  return __ffs(m) - 1;
}

// A window of D loads in flight per wave.  `next()` issues the loads of the
// next item of a source (items past the end read out of range, so every
// step issues the same loads and the waits the compiler inserts stay exact);
// `use` consumes items in order, D items behind the loads.
template <int D, class Frag>
struct Window {
  Frag buf[D + 1];  // D in flight and the one in use
  template <class NextF>
  __device__ __forceinline__ void prime(NextF next) {
#pragma unroll
    for (int j = 0; j < D; ++j) buf[j] = next();
  }
  // Step j of each pass of D + 1 steps: the free slot (j + D) mod (D + 1)
  // takes the next item's loads, then slot j is used.  A pass of D + 1 steps
  // ends with every slot back in its own registers.  With passes of D steps
  // the compiler copied the in-flight slots at the loop's back-edge, and a
  // copy waits for its loads: the window emptied on every pass.
  template <class NextF, class UseF>
  __device__ __forceinline__ void run(int n, NextF next, UseF use) {
    for (int base = 0; base < n; base += D + 1) {
#pragma unroll
      for (int j = 0; j <= D; ++j) {
        if (base + j < n) {
          buf[(j + D) % (D + 1)] = next();
          use(buf[j]);
        }
      }
    }
  }
  // The same for a window that has already used m items, m = S mod (D + 1):
  // its next item to use is in slot S.  Runs one after another continue the
  // one source without emptying the window in between.
  template <int S, class NextF, class UseF>
  __device__ __forceinline__ void run_rot(int n, NextF next, UseF use) {
    for (int base = 0; base < n; base += D + 1) {
#pragma unroll
      for (int j = 0; j <= D; ++j) {
        if (base + j < n) {
          buf[(S + j + D) % (D + 1)] = next();
          use(buf[(S + j) % (D + 1)]);
        }
      }
    }
  }
};

// -------------------------------------------------------- cross-CTA sync --

// Tagged words: a 32-bit payload with the call's epoch in the high half,
// stored and loaded as one 64-bit device-scope atomic.  A reader that finds
// this call's epoch in every word it needs has its data, with no separate
// flag, fence or counter between the writer and it.  Epochs only grow (the
// scratch is cleared whenever they restart), so a word from an earlier call
// never carries this call's tag.
__device__ __forceinline__ void st_tag(uint64_t* w, uint32_t v, uint32_t ep) {
  __hip_atomic_store(w, ((uint64_t)ep << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* w) {
  return __hip_atomic_load(const_cast<uint64_t*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t ep) { return (uint32_t)(w >> 32) == ep; }
// Two tagged words in one 16-byte device-scope load ({payload, tag, payload,
// tag}); each word carries its own tag, and an aligned 16-byte access is
// never split below 8 bytes.
__device__ __forceinline__ u32x4 ld_tag2(rsrc_t r, uint32_t word) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(word * 8u), 0, CP_SC1));
}

// Whether a wave polling since t0 gives up (wave-uniform): this call was
// aborted, an earlier call's error is unread (a handle in error fails fast
// instead of waiting out one deadline per call), or this wait passed its
// deadline, which aborts the call and records the first timeout.
__device__ __forceinline__ bool give_up(const Params& p, Bank* bk, unsigned long long t0, uint32_t wait_id,
                                        uint32_t seen, uint32_t target, uint32_t ep, uint32_t info) {
  const int lane = threadIdx.x & 63;
  uint32_t ab = 0;
  if (lane == 0) ab = __hip_atomic_load(&bk->abort_[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (lane == 1 && p.sticky) ab = __hip_atomic_load(&p.ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__ballot(ab != 0u)) return true;
  if (wall_clock64() - t0 > p.deadline_ticks) {
    if (lane == 0) {
      __hip_atomic_fetch_or(&bk->abort_[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t zero = 0;
      if (__hip_atomic_compare_exchange_strong(&p.ctl->error, &zero, (uint32_t)MOE_TAIL_ETIMEOUT, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        const uint32_t d[6] = {wait_id, blockIdx.x, seen, target, ep, info};
        for (int k = 0; k < 6; ++k)
          __hip_atomic_store(&p.ctl->diag[k], d[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return true;
  }
  return false;
}

// Wait until this workgroup's (SC1) stores have completed, then add n to *c.
__device__ __forceinline__ void publish(uint32_t* c, uint32_t n) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0 && n) __hip_atomic_fetch_add(c, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-uniform wait, polled by wave 0: counters c[k * stride] for k < n
// (n <= 64) all reach `target` (SUM false) or sum to at least `target` (SUM
// true).  Every wait has a deadline; a wait that passes it sets the abort
// word, which ends every other wait of the call.  Returns false when the call
// is aborted.
template <bool SUM>
__device__ __forceinline__ bool wait_cnt(const Params& p, Bank* bk, const uint32_t* c, int stride, int n,
                                         uint32_t target, bool stall, uint32_t* s_flag, uint32_t wait_id,
                                         uint32_t ep, uint32_t info) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint32_t ok = 1;
    const unsigned long long t0 = wall_clock64();
    while (true) {
      const uint32_t v = lane < n ? __hip_atomic_load(c + lane * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : (SUM ? 0u : 0xFFFFFFFFu);
      uint32_t seen;
      bool done;
      if (SUM) {
        int t = (int)v;
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        t += __shfl_xor(t, 8);
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        seen = (uint32_t)__builtin_amdgcn_readfirstlane(t);
        done = seen >= target;
      } else {
        done = __ballot(v < target) == 0;
        seen = done ? target : (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
      }
      if (done && !stall) break;
      if (give_up(p, bk, t0, wait_id, seen, target, ep, info)) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) *s_flag = ok;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return ok;
}

// Timeline build (-DMOE_TAIL_TIMELINE): thread 0 of every workgroup stamps
// the 100 MHz real-time counter at each phase edge of the last call.
#ifdef MOE_TAIL_TIMELINE
constexpr int TL_N = 32;
static __device__ unsigned long long g_timeline[1024 * TL_N];  // one per translation unit
#define TL(k)                                                                     \
  do {                                                                            \
    if (threadIdx.x == 0) g_timeline[blockIdx.x * TL_N + (k)] = wall_clock64(); \
  } while (0)
#define TL_ON 1
#else
#define TL(k) \
  do {        \
  } while (0)
#define TL_ON 0
#endif

struct FragA {  // one 16-byte weight load per lane
  u32x4 a;
};
struct FragU {  // MXFP4: up to 8 column groups of one unit, with their block-scale dwords
  u32x4 a[8];
  u32x4 s[2];
};
template <bool F8>
struct FragQB {  // one column group (one 16-byte load of MXFP4 codes, two of MXFP8) with its B fragments
  u32x4 a[F8 ? 2 : 1];
  uint32_t s;
  u32x4 b[4];
};
struct FragQB2 {  // MXFP4, two units of one slot: a column group's codes of both, one set of B fragments
  u32x4 a[2];
  uint32_t s[2];
  u32x4 b[4];
};
template <bool F8>
struct FragD {  // down: 2 column groups x both row blocks (x 2 halves for MXFP8), with their scale dwords
  u32x4 a[2][F8 ? 2 : 1][MAX_BLK];
  uint32_t s[MAX_BLK][2];
};
struct FragSD {
  u32x4 a[MAX_BLK];
};

template <bool WIDE>
struct SharedT {
  static constexpr int RW = WIDE ? MAX_RW : MAX_R;
  typedef typename std::conditional<WIDE, uint32_t, uint16_t>::type mask_t;  // a slot's users (one bit per row)
  uint32_t flags[8];
  uint32_t ep;
  double tmpd[NW];
  float tmpg[NW];             // shared gate: each wave's partial dot of a norm slice
  float rstd[RW];             // folded norm: each row's rstd
  float gsum[RW * NQ];        // shared gate: the slices' partial dots, per row
  float sgw[RW];              // shared gate: sigmoid(wg . xn) per row
  int wcnt[NW];
  int ucnt[NW];
  int last[MAX_ITEMS1];
  int16_t ids[MAX_P];
  float w[MAX_P];
  int16_t ci[MAX_P];
  uint32_t rowmask[MAX_E];
  int16_t eslot[MAX_E];
  int16_t slot_expert[MAX_P];
  mask_t slot_mask[MAX_P];
  int16_t slot_off[MAX_P + 1];
  int nslot;
  int nls;
  int16_t lsb[MAX_ITEMS1];  // shared blocks this workgroup finishes
  f32x4 red[2][NW][64];
};
constexpr int RED_FLOATS = 2 * NW * 64 * 4;  // floats in SharedT::red

// ------------------------------------------------------------------ kernel --

// WIDE: up to MAX_RW rows in one launch.  Where rows are MFMA columns (the
// router/shared K chunks, the shared down) a weight load feeds two 16-column
// tiles; an expert picked by more than 16 rows takes one slot per 16 of them
// (gate/up and down units stay one tile wide); the down phase stages the
// routed a in groups of slots that fit in LDS.
template <bool XL, bool RS, bool FEAT, bool F8, bool WIDE>
__device__ __forceinline__ void tail(const Params& p, SharedT<WIDE>& S, char* dyn) {
  static_assert(!WIDE || (!XL && !RS), "a wide launch reads xn from global scratch and sums router partials once");
  constexpr int PC = WIDE ? 32 : 16;  // columns per router/shared K-chunk partial tile
  const int tid = threadIdx.x, lane = tid & 63, cta = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int R = p.R, H = p.H, E = p.E, K = p.K, I = p.I, Is = p.Is, G = p.G;
  const int P = R * K;
  const int i16 = lane & 15, g = lane >> 4;  // MFMA row / column within 16, K-group
  const int n_rb = p.n_rb, n_sb = p.n_sb, S1 = p.S1, TC = p.TC;
  const int n_it = (n_rb + n_sb) * S1;
  const rsrc_t rs_xn = make_rsrc(p.xn, (uint32_t)(R * H * 2));
  const rsrc_t rs_xt = make_rsrc(p.xnt, (uint32_t)(R * H * 4));
  const rsrc_t rs_lt = make_rsrc(p.lgt, (uint32_t)(R * p.Ep * 8));
  const rsrc_t rs_pt = make_rsrc(p.part1, (uint32_t)(n_it * PC * 128));
  const rsrc_t rs_as = make_rsrc(p.a_s, (uint32_t)(R * Is * 2));
  const rsrc_t rs_ar = make_rsrc(p.a_r, (uint32_t)(P * I * 2));
  uint16_t* xl = (uint16_t*)dyn;  // [xrows][xs] staged activations; row xzero is zeros
  uint16_t* xc = (uint16_t*)dyn;  // [xrows][cs] this workgroup's K chunk of them (same space, earlier)
  const int xzero = p.xzero;

  TL(0);
  {  // Every 64-byte line of the kernel arguments at once: the first use of
     // each line would otherwise be a miss of its own, one after another.
    static_assert(sizeof(Params) <= 448, "the lines touched below cover the arguments");
    const char* kp = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    const uint32_t k0 = *(const uint32_t*)(kp + 64), k1 = *(const uint32_t*)(kp + 128), k2 = *(const uint32_t*)(kp + 192);
    const uint32_t k3 = *(const uint32_t*)(kp + 256), k4 = *(const uint32_t*)(kp + 320), k5 = *(const uint32_t*)(kp + 384);
    asm volatile("" ::"s"(k0), "s"(k1), "s"(k2), "s"(k3), "s"(k4), "s"(k5));
  }
  // This workgroup's output rows [h0, h0 + hn) of the combine (R hn <= NT: one
  // element per thread; an even width HR).  Their x and residual are loaded
  // now, so that the combine at the end does not wait for memory.
  const int HR = p.HR;
  const int h0 = min(H, cta * HR), hn = max(0, min(H, h0 + HR) - h0);
  const bool front = FEAT && p.attn;  // attention rows in place of x: x comes from the out_proj front below
  uint32_t cx, cr, cx2 = 0, cr2 = 0;  // (a wide launch has up to two elements per thread)
  {
    const int r = tid / max(hn, 1), hh = tid - r * max(hn, 1);
    const uint32_t off = tid < R * hn ? (uint32_t)(r * H + h0 + hh) * 2u : OOB;
    // no branches around these loads (an empty range reads zero), so that
    // nothing waits for them before the weights go out
    cx = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(p.x, p.x ? (uint32_t)(R * H * 2) : 0u), (int)off, 0, 0);
    cr = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(p.res ? p.res : p.gamma, p.res ? (uint32_t)(R * H * 2) : 0u),
                                              (int)off, 0, 0);
    if constexpr (WIDE) {
      const int q2 = tid + NT, r2 = q2 / max(hn, 1), hh2 = q2 - r2 * max(hn, 1);
      const uint32_t off2 = q2 < R * hn ? (uint32_t)(r2 * H + h0 + hh2) * 2u : OOB;
      cx2 = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(p.x, p.x ? (uint32_t)(R * H * 2) : 0u), (int)off2, 0, 0);
      cr2 = __builtin_amdgcn_raw_buffer_load_b16(
          make_rsrc(p.res ? p.res : p.gamma, p.res ? (uint32_t)(R * H * 2) : 0u), (int)off2, 0, 0);
    }
  }
  // ---- call epoch: every workgroup counts the calls it has started, so all
  // agree on it without a shared ticket (one launch = one call per workgroup).
  // The count is a read-modify-write atomic, like every other control word
  // that crosses workgroups or calls; nothing waits for its return until the
  // epoch is first needed.
  uint32_t epv = 0;
  if (tid == 0) {
    int z;  // an index the compiler cannot see is uniform: the atomic is issued as written, with no wait after it
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    epv = __hip_atomic_fetch_add(&p.ctl->cta_ep[cta][z], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < E) S.rowmask[tid] = 0u;
  if (tid == 0) S.flags[5] = 0u;  // set by a top-k wave whose logits poll gave up
  const bool stall = (p.debug_flags & MOE_TAIL_DEBUG_STALL) && cta == p.debug_block;

  // ---- router/shared source.  Item i = wi, wi + W1, ... (below) is K chunk
  // i % S1 of block i / S1 (router blocks of 16 experts, then shared blocks of
  // 8 gate + 8 up rows); S1 divides W1, so all of a workgroup's items share
  // chunk s1.
  // Wave w streams the chunk's 32-column groups [t01, t1e).
  const int s1 = cta % S1;
  const int TP1 = (TC + NW - 1) / NW, t01 = wave * TP1, t1e = min(TC, t01 + TP1);
  // With few rows the first nn1 workgroups (those that run the norm) take no
  // items: theirs would start last, behind the norm, and every router block
  // waits for its slowest chunk.  The others share the items round-robin (W1
  // of them; nn1 is a multiple of S1, so workgroup cta still takes chunk s1).
  const int W1 = G - p.nn1, wi = cta - p.nn1;
  const int nu1 = wi >= 0 && wi < n_it ? (n_it - 1 - wi) / W1 + 1 : 0;
  Window<D_BF, FragA> w1;
  int k1 = 0, t1 = t01;
  uint32_t roff1 = OOB;
  rsrc_t rs1 = make_rsrc(p.rw, (uint32_t)((size_t)E * H * 2));
  auto p1_unit = [&]() {  // decode item k1
    const int u = (wi + k1 * W1) / S1;
    int row;
    if (u < n_rb) {
      row = u * 16 + i16 < E ? u * 16 + i16 : -1;
      rs1 = make_rsrc(p.rw, (uint32_t)((size_t)E * H * 2));
    } else {
      const int sb = u - n_rb;
      row = i16 < 8 ? sb * 8 + i16 : Is + sb * 8 + (i16 - 8);
      rs1 = make_rsrc(p.ws13, (uint32_t)((size_t)2 * Is * H * 2));
    }
    roff1 = row >= 0 ? (uint32_t)(row * H + s1 * TC * 32 + g * 8) * 2u : OOB;
  };
  if (nu1) p1_unit();
  auto p1_next = [&]() {
    FragA f;
    const bool v = k1 < nu1 && t1 < t1e && roff1 != OOB;
    f.a = ld16<CP_W>(rs1, v ? roff1 + (uint32_t)t1 * 64u : OOB);
    if (++t1 == t01 + TP1) {
      t1 = t01;
      if (++k1 < nu1) p1_unit();
    }
    return f;
  };
  const bool is_norm = cta < (WIDE ? min(R, G / NQ) : R) * NQ;
  // Folded norm: this workgroup's K chunk of x, r and gamma (the first FCH
  // 16-byte vectors of each per thread) is loaded ahead of the weights, so
  // that it does not queue behind them; every load is issued (out-of-range
  // offsets where not needed) to keep the wait counts static.
  constexpr int FCH = 2;
  const bool fold = FEAT && p.fold && nu1;
  const int fc8n = TC * 4, fn8 = R * fc8n;  // 8-element vectors per chunk row, in all
  const rsrc_t frx = make_rsrc(p.x, (uint32_t)(R * H * 2));
  const rsrc_t frr = make_rsrc(p.res ? p.res : p.x, p.res ? (uint32_t)(R * H * 2) : 0u);
  const rsrc_t frg = make_rsrc(p.gamma, (uint32_t)(H * 2));
  u32x4 fx[FCH], fr[FCH], fg[FCH];
  auto fold_load = [&](int w, u32x4& xv, u32x4& rv, u32x4& gv) {
    const bool v = fold && w < fn8;
    const int r = w / fc8n, col = s1 * TC * 32 + (w - r * fc8n) * 8;
    xv = ld16<0>(frx, v ? (uint32_t)(r * H + col) * 2u : OOB);
    rv = ld16<0>(frr, v ? (uint32_t)(r * H + col) * 2u : OOB);
    gv = ld16<0>(frg, v ? (uint32_t)col * 2u : OOB);
  };
  auto fold_issue = [&]() {
    if constexpr (FEAT) {
      if (fold)
#pragma unroll
        for (int k = 0; k < FCH; ++k) fold_load(tid + k * NT, fx[k], fr[k], fg[k]);
    }
  };
  // ---- the out_proj front (attention rows in place of x): every workgroup
  // computes x of its slice, x[r][h] = bf16(sum_a attn[r][a] w_o[h][a]), and
  // publishes it as tagged pairs before its weights go out; the norm
  // workgroups read whole rows of it.  Every bf16 product is exact in double
  // and the sum is taken in double (thread (fh, fp) sums columns a = 8 (fp +
  // 16 j) .. + 7 of each K chunk for hidden row h0 + fh, then the 16 lanes of
  // a row in a fixed order), rounded to bf16 once, as the projection's
  // definition asks ("[AMD] integrate kimi k3 monokernel", K2 commit text,
  // Motivation and Modifications: out_proj in the same launch as the tail).
  if constexpr (FEAT) {
    if (front) {
      const int fh = tid >> 4, fpart = tid & 15, A = p.A;
      const rsrc_t rfa = make_rsrc(p.attn, (uint32_t)(R * A * 2));
      const rsrc_t rfw = make_rsrc(p.w_o, (uint32_t)((size_t)H * A * 2));
      uint16_t* const at = (uint16_t*)dyn;                      // [R][FRONT_AC] a K chunk of the attention rows
      uint16_t* const sx = (uint16_t*)&S.red[0][0][0];         // [R][32] this slice's x (tiles idle until later)
      double acc[MAX_R];
#pragma unroll
      for (int r = 0; r < MAX_R; ++r) acc[r] = 0.0;
      u32x4 fav[FRONT_AV], fwv[FRONT_WV];
      auto front_load = [&](int a0) {
        const int ac = min(FRONT_AC, A - a0), n8 = R * (ac / 8);
#pragma unroll
        for (int k = 0; k < FRONT_AV; ++k) {
          const int q = tid + k * NT, r = q / (ac / 8), c8 = q - r * (ac / 8);
          fav[k] = ld16<0>(rfa, q < n8 ? (uint32_t)(r * A + a0 + c8 * 8) * 2u : OOB);
        }
#pragma unroll
        for (int j = 0; j < FRONT_WV; ++j) {
          const int c8 = fpart + 16 * j;
          fwv[j] = ld16<0>(rfw, c8 * 8 < ac && fh < hn ? (uint32_t)((size_t)(h0 + fh) * A + a0 + c8 * 8) * 2u : OOB);
        }
      };
      front_load(0);
      for (int a0 = 0; a0 < A; a0 += FRONT_AC) {
        const int ac = min(FRONT_AC, A - a0), n8 = R * (ac / 8);
        if (a0) {
          __syncthreads();  // the previous chunk's readers are done
          front_load(a0);
        }
#pragma unroll
        for (int k = 0; k < FRONT_AV; ++k) {
          const int q = tid + k * NT, r = q / (ac / 8), c8 = q - r * (ac / 8);
          if (q < n8) *(u32x4*)(at + r * FRONT_AC + c8 * 8) = fav[k];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < FRONT_WV; ++j) {
          const int c8 = fpart + 16 * j;
          if (c8 * 8 < ac && fh < hn) {
            double wd[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              wd[2 * e] = (double)bf2f(fwv[j][e] & 0xFFFFu);
              wd[2 * e + 1] = (double)bf2f(fwv[j][e] >> 16);
            }
#pragma unroll
            for (int r = 0; r < MAX_R; ++r) {
              if (r < R) {
                const u32x4 av = lds16(at + r * FRONT_AC + c8 * 8);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  acc[r] = fma((double)bf2f(av[e] & 0xFFFFu), wd[2 * e], acc[r]);
                  acc[r] = fma((double)bf2f(av[e] >> 16), wd[2 * e + 1], acc[r]);
                }
              }
            }
          }
        }
      }
      // the 16 lanes of a hidden row: a prefix sum with row shifts, whose
      // lane 15 holds the total
#pragma unroll
      for (int r = 0; r < MAX_R; ++r) {
        if (r < R) {
          double v = acc[r];
          v += dpp_f64<0x111, 0xF>(v);
          v += dpp_f64<0x112, 0xF>(v);
          v += dpp_f64<0x114, 0xF>(v);
          v += dpp_f64<0x118, 0xF>(v);
          if (fpart == 15 && fh < hn) sx[r * 32 + fh] = (uint16_t)d2bf(v);
        }
      }
      if (tid == 0) S.ep = epv + 1u;  // the tags need the epoch here
      __syncthreads();
      const uint32_t epf = S.ep;
      const int r = tid / max(hn, 1), hh = tid - r * max(hn, 1);
      if (tid < R * hn) cx = sx[r * 32 + hh];
      const uint32_t xnext = (uint32_t)__shfl_down((int)cx, 1);  // column hh + 1 of the same row (hh even)
      if (tid < R * hn && (hh & 1) == 0) st_tag(p.xft + ((size_t)r * H + h0 + hh) / 2, cx | (xnext << 16), epf);
    }
  }
  // weights do not depend on the activations: their loads go out first,
  // except in the norm workgroups, whose row loads must not queue behind them
  fold_issue();
  if (!is_norm) w1.prime(p1_next);

  // ---- P0: fused residual add + RMSNorm; workgroup c < R*NQ owns slice c % NQ of row c / NQ
  // (in a wide launch, of rows c / NQ + j G / NQ, one after another)
  if (is_norm) for (int row = cta / NQ;; row += G / NQ) {
    const int q = cta % NQ, SL = H / NQ;
    const rsrc_t rx = make_rsrc(p.x + (size_t)row * H, (uint32_t)(H * 2));
    const rsrc_t rr = make_rsrc(p.res ? p.res + (size_t)row * H : p.x, p.res ? (uint32_t)(H * 2) : 0u);
    const rsrc_t rg = make_rsrc(p.gamma, (uint32_t)(H * 2));
    u32x4 xv[4], rv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // H <= 16384 = 4 x 512 x 8
      const int i = (k * NT + tid) * 8;
      xv[k] = ld16<0>(rx, !front && i < H ? (uint32_t)i * 2u : OOB);
      rv[k] = ld16<0>(rr, i < H ? (uint32_t)i * 2u : OOB);
    }
    // this workgroup's slice, loaded up front as well (8 elements per thread)
    const int i = q * SL + tid * 8;
    const bool sl = tid * 8 < SL;
    u32x4 x8 = ld16<0>(rx, !front && sl ? (uint32_t)i * 2u : OOB);
    const u32x4 r8 = ld16<0>(rr, sl ? (uint32_t)i * 2u : OOB);
    const u32x4 g8 = ld16<0>(rg, sl ? (uint32_t)i * 2u : OOB);
    if constexpr (FEAT) {
      if (front) {  // the row's x from every workgroup's slice of the front, polled until all is this call's
        const uint32_t epf = S.ep;
        const rsrc_t rxf = make_rsrc(p.xft + (size_t)row * (H / 2), (uint32_t)(H * 4));
        auto ld8 = [&](int e, bool v, bool& ok) -> u32x4 {  // 8 elements from two tagged-pair loads
          const u32x4 a = ld_tag2(rxf, v ? (uint32_t)(e / 2) : OOB / 8u);
          const u32x4 b = ld_tag2(rxf, v ? (uint32_t)(e / 2 + 2) : OOB / 8u);
          ok = ok && (!v || (a[1] == epf && a[3] == epf && b[1] == epf && b[3] == epf));
          return (u32x4){a[0], a[2], b[0], b[2]};
        };
        const unsigned long long t0 = wall_clock64();
        for (;;) {
          bool ok = true;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = (k * NT + tid) * 8;
            xv[k] = ld8(e, e < H, ok);
          }
          x8 = ld8(i, sl, ok);
          if (__syncthreads_and(ok && !stall)) break;
          if (tid < 64) {
            const bool gu = give_up(p, &p.ctl->bank[epf & 1], t0, 0, 0u, 1u, epf, 0u);
            if (tid == 0) S.flags[6] = gu;
          }
          __syncthreads();
          if (S.flags[6]) return;
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    u32x4 wg8 = {0u, 0u, 0u, 0u};  // shared gate slice
    if (FEAT && p.sgate) wg8 = ld16<0>(make_rsrc(p.sgate, (uint32_t)(H * 2)), sl ? (uint32_t)i * 2u : OOB);
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double h0 = bf2f(f2bf(bf2f(xv[k][c] & 0xFFFFu) + bf2f(rv[k][c] & 0xFFFFu)));
        const double h1 = bf2f(f2bf(bf2f(xv[k][c] >> 16) + bf2f(rv[k][c] >> 16)));
        ss = fma(h0, h0, ss);
        ss = fma(h1, h1, ss);
      }
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) S.tmpd[wave] = ss;
    if (tid == 0) S.ep = epv + 1u;  // the epoch atomic went out before the row loads
    __syncthreads();
    const uint32_t epn = S.ep;
    double tot = 0.0;
    for (int w = 0; w < NW; ++w) tot += S.tmpd[w];
    const double rstd = 1.0 / sqrt(tot / (double)H + p.eps);
    u32x4 nvs = {0u, 0u, 0u, 0u};  // this thread's 8 xn values (zeros outside the slice)
    if (sl) {
      u32x4 hv, nv;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t h0 = f2bf(bf2f(x8[c] & 0xFFFFu) + bf2f(r8[c] & 0xFFFFu));
        const uint32_t h1 = f2bf(bf2f(x8[c] >> 16) + bf2f(r8[c] >> 16));
        const uint32_t n0 = d2bf(((double)bf2f(h0) * rstd) * (double)bf2f(g8[c] & 0xFFFFu));
        const uint32_t n1 = d2bf(((double)bf2f(h1) * rstd) * (double)bf2f(g8[c] >> 16));
        hv[c] = h0 | (h1 << 16);
        nv[c] = n0 | (n1 << 16);
      }
      stc16(rs_xn, (uint32_t)(row * H + i) * 2u, nv);
      if (!(FEAT && p.fold))
#pragma unroll
        for (int c = 0; c < 4; ++c) st_tag(p.xnt + (size_t)(row * H + i) / 2 + c, nv[c], epn);
      if (p.res_out) *(u32x4*)(p.res_out + (size_t)row * H + i) = hv;
      nvs = nv;
    }
    if (FEAT && p.fold && q == 0 && tid == 0) st_tag(p.rstdt + row, __float_as_uint((float)rstd), epn);
    if (FEAT && p.sgate) {  // this slice's share of the gate's dot product: lanes, waves in order
      float gd = 0.f;
      if (sl) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          gd += bf2f(nvs[c] & 0xFFFFu) * bf2f(wg8[c] & 0xFFFFu);
          gd += bf2f(nvs[c] >> 16) * bf2f(wg8[c] >> 16);
        }
      }
      gd = wave_sum_f32(gd);
      if (lane == 0) S.tmpg[wave] = gd;
      __syncthreads();
      if (tid == 0) {
        float t = 0.f;
        for (int w = 0; w < NW; ++w) t += S.tmpg[w];
        st_tag(p.gpart + row * NQ + q, __float_as_uint(t), epn);
      }
    }
    if (!WIDE || row + G / NQ >= R) break;
    __syncthreads();  // the next row reuses S.tmpd and S.tmpg
  }
  if (FEAT && fold) {
    // folded norm: this chunk of bf16(h * gamma), from the inputs themselves
    // (no wait for the norm workgroups or the epoch; rstd is applied to the sums)
    auto put = [&](int w, const u32x4& xv, const u32x4& rv, const u32x4& gv) {
      if (w >= fn8) return;
      const int r = w / fc8n, c8 = w - r * fc8n;
      u32x4 hg;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t h0 = f2bf(bf2f(xv[c] & 0xFFFFu) + bf2f(rv[c] & 0xFFFFu));
        const uint32_t h1 = f2bf(bf2f(xv[c] >> 16) + bf2f(rv[c] >> 16));
        hg[c] = f2bf(bf2f(h0) * bf2f(gv[c] & 0xFFFFu)) | (f2bf(bf2f(h1) * bf2f(gv[c] >> 16)) << 16);
      }
      *(u32x4*)(xc + r * p.cs + c8 * 8) = hg;
    };
#pragma unroll
    for (int k = 0; k < FCH; ++k) put(tid + k * NT, fx[k], fr[k], fg[k]);
    for (int w = tid + FCH * NT; w < fn8; w += NT) {  // chunks beyond FCH vectors per thread
      u32x4 xv, rv, gv;
      fold_load(w, xv, rv, gv);
      put(w, xv, rv, gv);
    }
    for (int c = tid * 8; c < p.cs; c += NT * 8) *(u32x4*)(xc + xzero * p.cs + c) = (u32x4){0u, 0u, 0u, 0u};
    __syncthreads();
  }
  if (tid == 0) {
    uint32_t e1 = epv;
    asm volatile("" : "+v"(e1));  // keeps the wait for the atomic's return here
    S.ep = e1 + 1u;
  }
  __syncthreads();
  const uint32_t ep = S.ep;
  Bank* bk = &p.ctl->bank[ep & 1];
  if (cta == 0) {  // the next call's counters, with write-through (SC1) stores
    uint32_t* nb = (uint32_t*)&p.ctl->bank[(ep + 1) & 1];
    for (int i = tid * 16; i < BANK_WORDS; i += NT * 16)
      (void)__hip_atomic_exchange(nb + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (is_norm) {
    publish(&bk->normc[cta % NQ][0], WIDE ? (uint32_t)((R - 1 - cta / NQ) / (G / NQ) + 1) : 1u);
    w1.prime(p1_next);
  }
  TL(1);

  // Workgroup-uniform poll: attempt() loads tagged words, keeps their payloads
  // and reports whether all of this thread's words carry this call's tag; it
  // is repeated until every thread's do.  False when the call is aborted.
  auto poll_all = [&](auto attempt, uint32_t wait_id, uint32_t info, bool stl) -> bool {
    const unsigned long long t0 = wall_clock64();
    for (;;) {
      const bool ok = attempt();
      if (__syncthreads_and(ok && !stl)) return true;
      if (tid < 64) {
        const bool gu = give_up(p, bk, t0, wait_id, 0u, 1u, ep, info);
        if (tid == 0) S.flags[6] = gu;
      }
      __syncthreads();
      if (S.flags[6]) return false;
      __builtin_amdgcn_s_sleep(1);
    }
  };

  // ---- router/shared phase: stage this chunk of xn (tagged words written by
  // the norm workgroups), then the items' MFMA tiles
  if (!(FEAT && fold) && nu1) {
    const int CW = TC * 32, pr = CW / 4, np2 = R * pr;  // word pairs per row, in all
    if (!poll_all([&]() {
          bool ok = true;
          for (int w = tid; w < np2; w += NT) {
            const int r = w / pr, c = w - r * pr;
            const u32x4 v = ld_tag2(rs_xt, (uint32_t)(r * (H / 2) + s1 * (CW / 2) + 2 * c));
            ok = ok && v[1] == ep && v[3] == ep;
            *(uint2*)(xc + r * p.cs + 4 * c) = make_uint2(v[0], v[2]);
          }
          return ok;
        }, 0, 0, stall))
      return;
    TL(2);
    for (int c = tid * 8; c < p.cs; c += NT * 8) *(u32x4*)(xc + xzero * p.cs + c) = (u32x4){0u, 0u, 0u, 0u};
    __syncthreads();
  }
  TL(3);
  {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    int rb = 0, kk = 0, tt = 0;
    const int brow = (i16 < R ? i16 : xzero) * p.cs + g * 8;  // this lane's activation row in LDS
    const int brow1 = (16 + i16 < R ? 16 + i16 : xzero) * p.cs + g * 8;  // (wide: the second tile's)
    w1.run(nu1 * TP1, p1_next, [&](const FragA& f) {
      const int t = t01 + tt;
      const u32x4 b = lds16(xc + (t < t1e ? brow + t * 32 : xzero * p.cs));
      acc = mfma(as_bf16x8(f.a), as_bf16x8(b), acc);
      if constexpr (WIDE) {
        const u32x4 b1 = lds16(xc + (t < t1e ? brow1 + t * 32 : xzero * p.cs));
        acc1 = mfma(as_bf16x8(f.a), as_bf16x8(b1), acc1);
      }
      if (++tt == TP1) {  // item done: reduce the 8 waves' partials in wave order, store the chunk's partial
        tt = 0;
        const int it = wi + kk * W1;
        ++kk;
        if constexpr (WIDE) {  // both tiles at once (threads 256.. take the second), then a barrier
          S.red[0][wave][lane] = acc;
          S.red[1][wave][lane] = acc1;
          acc = (f32x4){0.f, 0.f, 0.f, 0.f};
          acc1 = (f32x4){0.f, 0.f, 0.f, 0.f};
          __syncthreads();
          const int tl = tid >> 8, l = (tid >> 2) & 63, qq = tid & 3;
          float v = 0.f;
          for (int w = 0; w < NW; ++w) v += S.red[tl][w][l][qq];
          const int row = 4 * (l >> 4) + qq, col = 16 * tl + (l & 15);
          if (col < R) st_tag(p.part1 + (it * PC + col) * 16 + row, __float_as_uint(v), ep);
          __syncthreads();
        } else {
          S.red[rb][wave][lane] = acc;
          acc = (f32x4){0.f, 0.f, 0.f, 0.f};
          __syncthreads();
          if (tid < 256) {
            const int l = tid >> 2, qq = tid & 3;
            float v = 0.f;
            for (int w = 0; w < NW; ++w) v += S.red[rb][w][l][qq];
            const int row = 4 * (l >> 4) + qq, col = l & 15;
            if (col < R) st_tag(p.part1 + (it * PC + col) * 16 + row, __float_as_uint(v), ep);
          }
          rb ^= 1;
        }
      }
    });
  }
  if (FEAT && p.fold) {  // every row's rstd (tagged words of the norm workgroups), while the partials drain
    if (!poll_all([&]() {
          if (tid >= R) return true;
          const uint64_t v = ld_tag(p.rstdt + tid);
          S.rstd[tid] = __uint_as_float((uint32_t)v);
          return tag_ok(v, ep);
        }, 0, 2, stall))
      return;
  }
  // count this workgroup's chunk arrivals; the last of a block's S1 chunks sums them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid < nu1) {
    const int u = (wi + tid * W1) / S1;
    const uint32_t old = __hip_atomic_fetch_add(&bk->unitc[u][0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.last[tid] = old == (uint32_t)(S1 - 1);
  }
  __syncthreads();
  {
    int nr = 0;
    for (int k = 0; k < nu1; ++k) {  // router blocks: logits = sum of the chunks in chunk order
      const int u = (wi + k * W1) / S1;
      if (!S.last[k] || u >= n_rb || RS) continue;
      if (tid < 16 * R) {
        const int col = tid >> 4, row = tid & 15;
        float t[NQ];
#pragma unroll
        for (int s = 0; s < NQ; ++s)
          if (s < S1) t[s] = __uint_as_float((uint32_t)ld_tag(p.part1 + ((u * S1 + s) * PC + col) * 16 + row));
        float v = 0.f;
#pragma unroll
        for (int s = 0; s < NQ; ++s)
          if (s < S1) v += t[s];
        if (FEAT && p.fold) v *= S.rstd[col];
        const int e = u * 16 + row;
        if (e < E) st_tag(p.lgt + col * p.Ep + e, __float_as_uint(v), ep);
      }
      ++nr;
    }
    (void)nr;
    // shared blocks: a = silu(gate) * up over the chunks summed in chunk order,
    // all of this workgroup's blocks at once (one round trip for the partials)
    if (tid == 0) {
      int ns = 0;
      for (int k = 0; k < nu1; ++k) {
        const int u = (wi + k * W1) / S1;
        if (S.last[k] && u >= n_rb) S.lsb[ns++] = (int16_t)(u - n_rb);
      }
      S.nls = ns;
    }
    __syncthreads();
    const int ns = S.nls;
    for (int idx = tid; idx < ns * 8 * R; idx += NT) {
      const int k = idx / (8 * R), rc = idx - k * 8 * R, col = rc >> 3, row = rc & 7;
      const int sb = S.lsb[k], u = n_rb + sb;
      float tg[NQ], tu[NQ];
#pragma unroll
      for (int s = 0; s < NQ; ++s)
        if (s < S1) {
          tg[s] = __uint_as_float((uint32_t)ld_tag(p.part1 + ((u * S1 + s) * PC + col) * 16 + row));
          tu[s] = __uint_as_float((uint32_t)ld_tag(p.part1 + ((u * S1 + s) * PC + col) * 16 + row + 8));
        }
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int s = 0; s < NQ; ++s)
        if (s < S1) {
          gs += tg[s];
          us += tu[s];
        }
      if (FEAT && p.fold) {
        gs *= S.rstd[col];
        us *= S.rstd[col];
      }
      const float a = gs / (1.f + __expf(-gs)) * us;
      stc2(rs_as, (uint32_t)(col * Is + sb * 8 + row) * 2u, f2bf(a));
    }
    if (ns) publish(&bk->shared[0], (uint32_t)ns);
  }
  TL(4);

  // ---- all of xn, for the routed gate/up phase
  if (!wait_cnt<false>(p, bk, &bk->normc[0][0], 16, NQ, (uint32_t)R, stall && !nu1, &S.flags[1], 0, ep, 1)) return;
  if constexpr (XL) {  // stage xn [R][H] -> LDS rows of stride xs; row xzero stays zero
    const int n8 = R * H / 8;
    for (int base = 0; base < n8; base += NT * 8) {
      u32x4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e8 = base + k * NT + tid;
        v[k] = ld16<CP_SC1>(rs_xn, e8 < n8 ? (uint32_t)e8 * 16u : OOB);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e8 = base + k * NT + tid;
        if (e8 < n8) {
          const int r = (e8 * 8) / H, c = (e8 * 8) % H;
          *(u32x4*)(xl + r * p.xs + c) = v[k];
        }
      }
    }
    for (int c = tid * 8; c < p.xs; c += NT * 8) *(u32x4*)(xl + xzero * p.xs + c) = (u32x4){0u, 0u, 0u, 0u};
  }

  // ---- top-k on every workgroup (identical inputs, identical result).  Lane l
  // holds experts 8l..8l+7 as (key, 7 - j) pairs sorted once in descending
  // order; a round takes the wave-wide largest head, which on equal keys is the
  // lowest lane and within it the lowest j: the lower expert id ("glm53:
  // Long-context indexer ...", PR 85 commit row 9: ID order on ties)
  // With few rows x chunks, each workgroup sums the router chunks itself (in
  // chunk order, the same sums as above) into LDS: no last-arriver hop.
  float* const lgs = (float*)&S.red[0][0][0];  // [R][E]; the reduction tiles are idle here
  if constexpr (RS) {
    const int E4 = (E + 3) >> 2;
    if (!poll_all([&]() {
          bool ok = true;
          for (int q = tid; q < R * E4; q += NT) {  // 4 experts of one row per thread
            const int r = q / E4, e = 4 * (q - r * E4), u = e >> 4, row = e & 15;
            u32x4 t[NQ][2];
#pragma unroll
            for (int s = 0; s < NQ; ++s)
              if (s < S1)
#pragma unroll
                for (int j = 0; j < 2; ++j) t[s][j] = ld_tag2(rs_pt, (uint32_t)(((u * S1 + s) * 16 + r) * 16 + row + 2 * j));
            float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NQ; ++s)
              if (s < S1)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  ok = ok && t[s][j >> 1][2 * (j & 1) + 1] == ep;
                  v[j] += __uint_as_float(t[s][j >> 1][2 * (j & 1)]);
                }
            const float sc = FEAT && p.fold ? S.rstd[r] : 1.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (e + j < E) lgs[r * E + e + j] = v[j] * sc;
          }
          return ok;
        }, 1, 0, false))
      return;
  }
  TL(5);
  // The shared expert's down weights for this workgroup's hidden rows do not
  // depend on the routing: their first loads go out here, while the memory
  // system is quiet, and stay in registers until the down phase uses them.
  const int nblk = (hn + 15) / 16;
  const int Cs = Is / 32, CPs = (Cs + NW - 1) / NW, c0s = wave * CPs;
  const rsrc_t rqs = make_rsrc(p.ws2 + (size_t)h0 * Is, (uint32_t)(hn * Is * 2));
  int cse = c0s;
  auto sd_next = [&]() {  // every load is issued (out of range where not needed): the waits stay counted
    FragSD f;
#pragma unroll
    for (int bl = 0; bl < MAX_BLK; ++bl) {
      const int hh = 16 * bl + i16;
      const bool v = cse < c0s + CPs && cse < Cs && bl < nblk && hh < hn;
      f.a[bl] = ld16<CP_W>(rqs, v ? (uint32_t)(hh * Is + cse * 32 + g * 8) * 2u : OOB);
    }
    ++cse;
    return f;
  };
  // (With the optional steps, whose kernels hold more registers, only at 1-2
  // rows; at more rows they prime it in the down phase, measured faster there.)
  const bool wse = !FEAT || R <= 2;
  Window<2, FragSD> ws;
  if (wse) ws.prime(sd_next);
  for (int r = wave; r < R; r += NW) {
    const int e0 = 8 * lane;
    float lg[8];
    if constexpr (RS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) lg[j] = e0 + j < E ? lgs[r * E + e0 + j] : 0.f;
    } else {  // this row's tagged logits, polled by this wave alone
      const unsigned long long t0 = wall_clock64();
      bool failed = false;
      for (;;) {
        bool ok = true;
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = ld_tag2(rs_lt, e0 < E ? (uint32_t)(r * p.Ep + e0 + 2 * j) : OOB / 8u);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          ok = ok && (e0 + j >= E || v[j >> 1][2 * (j & 1) + 1] == ep);
          lg[j] = __uint_as_float(v[j >> 1][2 * (j & 1)]);
        }
        if (__ballot(!ok) == 0) break;
        if (give_up(p, bk, t0, 1, 0u, 1u, ep, (uint32_t)r)) {
          failed = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (failed) {
        if (lane == 0) S.flags[5] = 1u;
        continue;
      }
    }
    uint64_t qv[8];
    if (p.scoring == MOE_TAIL_SOFTMAX) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        qv[j] = ((uint64_t)(e0 + j < E ? ord_key(lg[j]) : 0u) << 32) | (uint32_t)(7 - j);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + j;
        const float kf = 1.f / (1.f + __expf(-lg[j])) + (e < E ? p.bias[e] : 0.f);
        qv[j] = ((uint64_t)(e < E ? ord_key(kf) : 0u) << 32) | (uint32_t)(7 - j);
      }
    }
#define MT_CX(a, b)                    \
  {                                    \
    const uint64_t x_ = qv[a], y_ = qv[b]; \
    const bool s_ = y_ > x_;           \
    qv[a] = s_ ? y_ : x_;              \
    qv[b] = s_ ? x_ : y_;              \
  }
    MT_CX(0, 1) MT_CX(2, 3) MT_CX(4, 5) MT_CX(6, 7)
    MT_CX(0, 2) MT_CX(1, 3) MT_CX(4, 6) MT_CX(5, 7)
    MT_CX(1, 2) MT_CX(5, 6)
    MT_CX(0, 4) MT_CX(1, 5) MT_CX(2, 6) MT_CX(3, 7)
    MT_CX(2, 4) MT_CX(3, 5)
    MT_CX(1, 2) MT_CX(3, 4) MT_CX(5, 6)
#undef MT_CX
    if (FEAT && p.n_group > 1) {
      // group-limited routing: lanes hold 8 consecutive experts, so a group is
      // gl consecutive lanes [gb, gb + gl) (gl = E / n_group / 8, any value).
      // Each lane merges the own top-2 of the group's other lanes, read in gl - 1
      // rotations that never leave the group, into its pair; every lane of the
      // group then holds the group's two largest keys (max/min merges, so the
      // result does not depend on the order).  The groups are ranked by the
      // pair's sum in topk_group rounds (equal sums: the lowest lane, i.e. the
      // lower group), and the experts of the other groups drop out.
      const int gl = E / p.n_group / 8;
      const int gb = (lane / gl) * gl, li = lane - gb;
      const float o1 = key_float((uint32_t)(qv[0] >> 32)), o2 = key_float((uint32_t)(qv[1] >> 32));
      float a1 = o1, a2 = o2;
      for (int s = 1; s < gl; ++s) {
        const int src = gb + (li + s < gl ? li + s : li + s - gl);
        const float b1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(o1)));
        const float b2 = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(o2)));
        const float n2 = a1 >= b1 ? fmaxf(b1, a2) : fmaxf(a1, b2);
        a1 = fmaxf(a1, b1);
        a2 = n2;
      }
      uint32_t gk = e0 < E ? ord_key(a1 + a2) : 0u;
      bool kept = false;
      for (int t = 0; t < p.topk_group; ++t) {
        const uint32_t m = wave_max_u32(gk);
        const int wl = __ffsll((unsigned long long)__ballot(gk == m)) - 1;
        if (lane / gl == wl / gl) {
          kept = true;
          gk = 0u;
        }
      }
      if (!kept) {
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[j] = 0;
      }
    }
    int myid = 0;
    for (int k = 0; k < K; ++k) {
      const uint32_t head = (uint32_t)(qv[0] >> 32);
      const uint32_t m = wave_max_u32(head);
      const int wl = __ffsll((unsigned long long)__ballot(head == m)) - 1;
      const int id = 8 * wl + 7 - __builtin_amdgcn_readlane((int)(uint32_t)qv[0], wl);
      if (lane == wl) {
#pragma unroll
        for (int v = 0; v < 7; ++v) qv[v] = qv[v + 1];
        qv[7] = 0;
      }
      if (lane == k) myid = id;
    }
    // lane k < K: pick k's logit, read from the lane that holds it
    float lsel = 0.f;
    const int src = (myid >> 3) << 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(lg[j])));
      if ((myid & 7) == j) lsel = v;
    }
    const float lmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lsel)));  // pick 0
    float t = 0.f;
    if (lane < K) t = p.scoring == MOE_TAIL_SOFTMAX ? __expf(lsel - lmax) : 1.f / (1.f + __expf(-lsel));
    const float sum = wave_sum_f32(t);
    if (lane < K) {
      S.ids[r * K + lane] = (int16_t)myid;
      S.w[r * K + lane] = t / sum * p.rscale;
      atomicOr(&S.rowmask[myid], 1u << r);
    }
  }
  __syncthreads();
  if (S.flags[5]) return;  // a logits poll gave up: the call is aborted
  TL(6);

  // ---- de-duplication: one slot per distinct expert, in expert order, with
  // the rows that picked it; users of slot d are rows [slot_off[d], slot_off[d+1]) of a
  {
    const uint32_t m = tid < E ? S.rowmask[tid] : 0u;
    const uint64_t bal = __ballot(m != 0u);
    const int users = __popc(m);  // <= 16 (wide: <= 32)
    int pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < (WIDE ? 6 : 5); ++b) {
      const uint64_t bb = __ballot((users >> b) & 1);
      pre += __popcll(bb & lanes_below()) << b;
      tot += __popcll(bb) << b;
    }
    // slots before this expert's in the wave (wide: one slot per 16 users)
    int spre = 0;
    if constexpr (WIDE) {
      const int nse = (users + 15) >> 4;
      const uint64_t b0 = __ballot(nse & 1), b1 = __ballot(nse >> 1);
      spre = __popcll(b0 & lanes_below()) + 2 * __popcll(b1 & lanes_below());
      if (lane == 0) S.wcnt[wave] = __popcll(b0) + 2 * __popcll(b1);
    } else {
      if (lane == 0) S.wcnt[wave] = __popcll(bal);
    }
    if (lane == 0) S.ucnt[wave] = tot;
    __syncthreads();
    int sb = 0, ub = 0, ns = 0, nus = 0;
    for (int w = 0; w < NW; ++w) {
      const int a = S.wcnt[w], b = S.ucnt[w];
      if (w < wave) {
        sb += a;
        ub += b;
      }
      ns += a;
      nus += b;
    }
    if (m) {
      const int slot = sb + (WIDE ? spre : __popcll(bal & lanes_below()));
      S.slot_expert[slot] = (int16_t)tid;
      S.slot_mask[slot] = (typename SharedT<WIDE>::mask_t)m;
      S.slot_off[slot] = (int16_t)(ub + pre);
      S.eslot[tid] = (int16_t)slot;
      if (WIDE && users > 16) {  // the first 16 users (in row order), then the rest
        const uint32_t lo = m & ((1u << nth_bit(m, 16)) - 1u);
        S.slot_mask[slot] = lo;
        S.slot_expert[slot + 1] = (int16_t)tid;
        S.slot_mask[slot + 1] = m & ~lo;
        S.slot_off[slot + 1] = (int16_t)(ub + pre + 16);
      }
    }
    if (tid == 0) {
      S.nslot = ns;
      S.slot_off[ns] = (int16_t)nus;
    }
    __syncthreads();
  }
  const int D = S.nslot;
  if (cta == 0) {
    for (int q = tid; q < P; q += NT) {
      if (p.topk_ids) p.topk_ids[q] = S.ids[q];
      if (p.topk_w) p.topk_w[q] = S.w[q];
    }
    if (p.dbg_logits) {
      for (int q = tid; q < R * E; q += NT)
        p.dbg_logits[q] = RS ? lgs[q] : __uint_as_float((uint32_t)ld_tag(p.lgt + (q / E) * p.Ep + q % E));
      if (RS) __syncthreads();  // the routed phase reuses these LDS tiles
    }
  }
  TL(7);

  // ---- P2: routed gate/up units (slot, 8 intermediate indices), waves split K
  {
    // DU: with activations from global memory (MXFP4), a work unit is two
    // units (blocks b, b + 1 of one slot) whose two weight tiles share each
    // activation load, which doubles the weight bytes a wave keeps in flight
    constexpr bool DU = !XL && !F8;
    const int UB = I / 8, UW = DU ? UB / 2 : UB, n_p2 = D * UW;
    const int T2 = H / 128, TP2 = (T2 + NW - 1) / NW, t02 = wave * TP2;
    // Units go round-robin from workgroup off2 on: the workgroups before it
    // reach this phase last (the norm's, or those with one more router/shared
    // item), so the units left over after whole rounds go to early ones.  off2
    // is a multiple of 8, which keeps each unit on the same XCD.
    int off2 = p.nn1 ? p.nn1 + n_it % (G - p.nn1) : max(R * NQ, n_it % G);
    off2 = (off2 & ~7) % G;
    const int u0 = cta >= off2 ? cta - off2 : cta + G - off2;
    const int nu2 = u0 < n_p2 ? (n_p2 - 1 - u0) / G + 1 : 0;
    // codes per expert: MXFP4 packs two per byte, MXFP8 one
    const int RB13 = F8 ? H : H / 2;
    const size_t S13 = (size_t)2 * I * RB13, S13s = (size_t)2 * I * (H / 32);
    int rb = 0;
    // end of unit u: reduce the 8 waves' partials in wave order; a = silu(gate) * up
    auto p2_reduce = [&](f32x4 acc, int u) {
      const int d = u / UB, bb = u - d * UB;
      const int m = __popc((uint32_t)S.slot_mask[d]);
      S.red[rb][wave][lane] = acc;
      __syncthreads();
      if (tid < 128) {
        const int l = tid >> 2, qq = tid & 3;
        float gs = 0.f, us = 0.f;
        for (int w = 0; w < NW; ++w) {
          gs += S.red[rb][w][l][qq];
          us += S.red[rb][w][l + 32][qq];
        }
        const int ii = 4 * (l >> 4) + qq, col = l & 15;
        const float a = gs / (1.f + __expf(-gs)) * us;
        if (col < m) stc2(rs_ar, (uint32_t)((S.slot_off[d] + col) * I + bb * 8 + ii) * 2u, f2bf(a));
      }
      rb ^= 1;
    };
    if constexpr (XL) {
      // A frag is one part (up to 8 column groups) of a unit: its code loads and
      // the block-scale dwords of those column groups (lane (i16, g) loads dwords
      // tb .. tb+7 of its row; column group tb + tt uses dword tt, byte g), so a
      // unit costs one or two scale loads instead of one per column group.
      // an MXFP8 column group takes two 16-byte loads, so a frag holds 4 of them
      constexpr int CPF = F8 ? 4 : 8;
      const int NP = (TP2 + CPF - 1) / CPF;
      int k2 = 0, q2 = 0;
      auto p2_next = [&]() {
        FragU f;
        const bool v = k2 < nu2;
        const int u = u0 + (v ? k2 : 0) * G, d = u / UB, b = u - d * UB;
        const int e = __builtin_amdgcn_readfirstlane(S.slot_expert[d]);  // uniform: scalar descriptors
        const rsrc_t rq = make_rsrc(p.w13q + e * S13, (uint32_t)S13);
        const rsrc_t rs = make_rsrc(p.w13s + e * S13s, (uint32_t)S13s);
        const int wrow = i16 < 8 ? b * 8 + i16 : I + b * 8 + (i16 - 8);
        const int tb = t02 + CPF * q2, np = min(CPF, TP2 - CPF * q2);
        // unit-blocked MXFP4 layout: unit b's column group c is 1 KB, lane-ordered
        const bool sh = !F8 && p.shuf;
        const uint32_t qoff = sh ? (uint32_t)(b * T2 * 1024 + lane * 16) : (uint32_t)(wrow * RB13 + g * (F8 ? 32 : 16));
        const uint32_t soff = (uint32_t)(wrow * (H / 32) + tb * 4), cst = sh ? 1024u : 64u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = F8 ? j >> 1 : j;
          const uint32_t o = F8 ? (uint32_t)(tb + t) * 128u + (uint32_t)(j & 1) * 16u : (uint32_t)(tb + t) * cst;
          f.a[j] = ld16<CP_W>(rq, (v && t < np && tb + t < T2) ? qoff + o : OOB);
        }
        f.s[0] = ld16<CP_W>(rs, v ? soff : OOB);
        f.s[1] = ld16<CP_W>(rs, (v && np > 4) ? soff + 16u : OOB);
        if (++q2 == NP) {
          q2 = 0;
          ++k2;
        }
        return f;
      };
      Window<1, FragU> w2;
      w2.prime(p2_next);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      int kk = 0, qc = 0;
      if (nu2 && TL_ON) TL(13);
      w2.run(nu2 * NP, p2_next, [&](const FragU& f) {
        const int u = u0 + kk * G, d = u / UB;
        const uint32_t mask = S.slot_mask[d];
        const int brow = (i16 < __popc(mask) ? nth_bit(mask, i16) : xzero) * p.xs + g * 32;
        const int tb = t02 + CPF * qc, np = min(CPF, TP2 - CPF * qc);
#pragma unroll
        for (int tt = 0; tt < CPF; ++tt) {
          if (tt < np) {
            const int t = tb + tt;
            const float sc = e8m0f((f.s[tt >> 2][tt & 3] >> (8 * g)) & 0xFFu);
            u32x4 bq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) bq[q] = lds16(xl + (t < T2 ? brow + t * 128 + 8 * q : xzero * p.xs));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bf16x8 aq = F8 ? fp8x8(f.a[2 * tt + (q >> 1)][2 * (q & 1)], f.a[2 * tt + (q >> 1)][2 * (q & 1) + 1], sc)
                                   : fp4x8(f.a[tt][q], sc);
              acc = mfma(aq, as_bf16x8(bq[q]), acc);
            }
          }
        }
        if (++qc == NP) {
          qc = 0;
          p2_reduce(acc, u);
          acc = (f32x4){0.f, 0.f, 0.f, 0.f};
          if (kk < 8) TL(14 + kk);
          ++kk;
        }
      });
    } else {
      // activations from global memory: one column group per frag, with its B fragments
      if constexpr (DU) {
        // work unit w = (slot d, pair bp): units (d, 2 bp) and (d, 2 bp + 1)
        int k2 = 0, t2 = t02;
        rsrc_t rq2 = rs_xn, rsc2 = rs_xn;
        uint32_t qoff0 = 0, qoff1 = 0, soff0 = 0, soff1 = 0, boff = OOB, qst = 64u;
        auto p2_unit = [&]() {
          const int w = u0 + k2 * G, d = w / UW, b = 2 * (w - d * UW);
          const int e = __builtin_amdgcn_readfirstlane(S.slot_expert[d]);  // uniform: scalar descriptors
          rq2 = make_rsrc(p.w13q + e * S13, (uint32_t)S13);
          rsc2 = make_rsrc(p.w13s + e * S13s, (uint32_t)S13s);
          const int wrow0 = i16 < 8 ? b * 8 + i16 : I + b * 8 + (i16 - 8), wrow1 = wrow0 + 8;
          const bool sh = p.shuf;  // unit-blocked MXFP4 layout
          qoff0 = sh ? (uint32_t)(b * T2 * 1024 + lane * 16) : (uint32_t)(wrow0 * RB13 + g * 16);
          qoff1 = sh ? qoff0 + (uint32_t)(T2 * 1024) : (uint32_t)(wrow1 * RB13 + g * 16);
          qst = sh ? 1024u : 64u;
          soff0 = (uint32_t)(wrow0 * (H / 32));
          soff1 = (uint32_t)(wrow1 * (H / 32));
          const uint32_t mask = S.slot_mask[d];
          boff = i16 < __popc(mask) ? (uint32_t)(nth_bit(mask, i16) * H + g * 32) * 2u : OOB;
        };
        if (nu2) p2_unit();
        auto p2_next = [&]() {
          FragQB2 f;
          const bool v = k2 < nu2 && t2 < T2;
          f.a[0] = ld16<CP_W>(rq2, v ? qoff0 + (uint32_t)t2 * qst : OOB);
          f.a[1] = ld16<CP_W>(rq2, v ? qoff1 + (uint32_t)t2 * qst : OOB);
          f.s[0] = ld4<CP_W>(rsc2, v ? soff0 + (uint32_t)t2 * 4u : OOB);
          f.s[1] = ld4<CP_W>(rsc2, v ? soff1 + (uint32_t)t2 * 4u : OOB);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            f.b[q] = ld16<CP_SC1>(rs_xn, (v && boff != OOB) ? boff + (uint32_t)(t2 * 256 + 16 * q) : OOB);
          if (++t2 == t02 + TP2) {
            t2 = t02;
            if (++k2 < nu2) p2_unit();
          }
          return f;
        };
        Window<D_FP4_G, FragQB2> w2;
        w2.prime(p2_next);
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        int kk = 0, tt = 0;
        if (nu2 && TL_ON) TL(13);
        w2.run(nu2 * TP2, p2_next, [&](const FragQB2& f) {
          const float sc0 = e8m0f((f.s[0] >> (8 * g)) & 0xFFu), sc1 = e8m0f((f.s[1] >> (8 * g)) & 0xFFu);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc0 = mfma(fp4x8(f.a[0][q], sc0), as_bf16x8(f.b[q]), acc0);
            acc1 = mfma(fp4x8(f.a[1][q], sc1), as_bf16x8(f.b[q]), acc1);
          }
          if (++tt == TP2) {
            tt = 0;
            const int w = u0 + kk * G, d = w / UW, u = d * UB + 2 * (w - d * UW);
            p2_reduce(acc0, u);
            p2_reduce(acc1, u + 1);
            acc0 = (f32x4){0.f, 0.f, 0.f, 0.f};
            acc1 = (f32x4){0.f, 0.f, 0.f, 0.f};
            if (kk < 8) TL(14 + kk);
            ++kk;
          }
        });
      } else {
        int k2 = 0, t2 = t02;
        rsrc_t rq2 = rs_xn, rsc2 = rs_xn;
        uint32_t qoff = 0, soff = 0, boff = OOB, qst = F8 ? 128u : 64u;
        auto p2_unit = [&]() {
          const int u = u0 + k2 * G, d = u / UB, b = u - d * UB;
          const int e = __builtin_amdgcn_readfirstlane(S.slot_expert[d]);  // uniform: scalar descriptors
          rq2 = make_rsrc(p.w13q + e * S13, (uint32_t)S13);
          rsc2 = make_rsrc(p.w13s + e * S13s, (uint32_t)S13s);
          const int wrow = i16 < 8 ? b * 8 + i16 : I + b * 8 + (i16 - 8);
          const bool sh = !F8 && p.shuf;  // unit-blocked MXFP4 layout
          qoff = sh ? (uint32_t)(b * T2 * 1024 + lane * 16) : (uint32_t)(wrow * RB13 + g * (F8 ? 32 : 16));
          qst = sh ? 1024u : (F8 ? 128u : 64u);
          soff = (uint32_t)(wrow * (H / 32));
          const uint32_t mask = S.slot_mask[d];
          boff = i16 < __popc(mask) ? (uint32_t)(nth_bit(mask, i16) * H + g * 32) * 2u : OOB;
        };
        if (nu2) p2_unit();
        auto p2_next = [&]() {
          FragQB<F8> f;
          const bool v = k2 < nu2 && t2 < T2;
#pragma unroll
          for (int j = 0; j < (F8 ? 2 : 1); ++j)
            f.a[j] = ld16<CP_W>(rq2, v ? qoff + (uint32_t)t2 * qst + (uint32_t)j * 16u : OOB);
          f.s = ld4<CP_W>(rsc2, v ? soff + (uint32_t)t2 * 4u : OOB);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            f.b[q] = ld16<CP_SC1>(rs_xn, (v && boff != OOB) ? boff + (uint32_t)(t2 * 256 + 16 * q) : OOB);
          if (++t2 == t02 + TP2) {
            t2 = t02;
            if (++k2 < nu2) p2_unit();
          }
          return f;
        };
        Window<D_FP4_G, FragQB<F8>> w2;
        w2.prime(p2_next);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        int kk = 0, tt = 0;
        if (nu2 && TL_ON) TL(13);
        w2.run(nu2 * TP2, p2_next, [&](const FragQB<F8>& f) {
          const float sc = e8m0f((f.s >> (8 * g)) & 0xFFu);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bf16x8 aq = F8 ? fp8x8(f.a[(q >> 1) & (F8 ? 1 : 0)][2 * (q & 1)], f.a[(q >> 1) & (F8 ? 1 : 0)][2 * (q & 1) + 1], sc)
                                 : fp4x8(f.a[0][q], sc);
            acc = mfma(aq, as_bf16x8(f.b[q]), acc);
          }
          if (++tt == TP2) {
            tt = 0;
            p2_reduce(acc, u0 + kk * G);
            acc = (f32x4){0.f, 0.f, 0.f, 0.f};
            if (kk < 8) TL(14 + kk);
            ++kk;
          }
        });
      }
    }
    if (nu2) publish(&bk->routed[cta % NRC][0], (uint32_t)(DU ? 2 * nu2 : nu2));
  }
  TL(8);

  // ---- P3: down projections for this workgroup's hidden rows, then combine
  const int CI = I / 32, TI = (CI + 3) / 4;
  const int nsl = D > wave ? (D - wave + NW - 1) / NW : 0;
  const int RB2 = F8 ? I : I / 2;  // down code bytes per hidden row
  const size_t S2 = (size_t)H * RB2, S2s = (size_t)H * CI;
  uint16_t* al = (uint16_t*)dyn;                // [P + 1][as] routed a; row azero is zeros
  uint16_t* asl = (uint16_t*)(dyn + p.off_as);  // [R + 1][ss] shared a; row szero is zeros
  float* s_outp = (float*)(dyn + p.off_outp);   // [P][HR]
  float* s_shp = (float*)(dyn + p.off_shp);     // [NW][R][HR]
  const int azero = p.azero, szero = p.szero;
  // source: frags of 2 column groups (of 128 I-elements) of slot j3 (slot
  // d = wave + NW * j3), both 16-row blocks, with their block scales: lane
  // (i16, g) needs scale byte 4 t3 + g of its row for column group t3, and
  // loads the dword that holds it.  Every load is issued (out-of-range ones
  // read zero without a memory access), so the compiler counts them exactly.
  const int NP3 = (TI + 1) / 2;
  const int s3r = (h0 * CI) & 3;  // slice start mod 4 (expert strides H CI are multiples of 4)
  int j3 = 0, q3 = 0;
  auto p3_next = [&]() {
    FragD<F8> f;
    const bool v = j3 < nsl && hn > 0;
    const int e = v ? __builtin_amdgcn_readfirstlane(S.slot_expert[wave + NW * j3]) : 0;  // uniform
    // scale bytes from a 4-byte aligned base at or below the slice start; the
    // dword loads stay inside the array (its size is a multiple of 4)
    const size_t so = (size_t)e * S2s + (size_t)h0 * CI, sa = so & ~(size_t)3;
    const uint32_t sr = (uint32_t)(so - sa);
    const rsrc_t rq = make_rsrc_u(p.w2q + e * S2 + (size_t)h0 * RB2, (uint32_t)(hn * RB2));
    const rsrc_t rs = make_rsrc_u(p.w2s + sa, (uint32_t)((size_t)E * H * CI - sa));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int t3 = 2 * q3 + t, c = 4 * t3 + g;
#pragma unroll
      for (int bl = 0; bl < MAX_BLK; ++bl) {
        const int hh = 16 * bl + i16;
        const bool ok = v && t3 < TI && bl < nblk && hh < hn && c < CI;
#pragma unroll
        for (int j = 0; j < (F8 ? 2 : 1); ++j)
          f.a[t][j][bl] = ld16<CP_W>(rq, ok ? (uint32_t)(hh * RB2 + c * (F8 ? 32 : 16) + j * 16) : OOB);
        f.s[bl][t] = ld4<CP_W>(rs, ok ? (sr + (uint32_t)(hh * CI + c)) & ~3u : OOB);
      }
    }
    if (++q3 == NP3) {
      q3 = 0;
      ++j3;
    }
    return f;
  };
  // the shared gate of every row: the norm slices' partial dots, long written
  // by now, summed in slice order (before the down weights' loads go out)
  if (FEAT && p.sgate && Is > 0 && hn > 0) {
    if (!poll_all([&]() {
          bool ok = true;
          if (tid < R * NQ) {
            const uint64_t w = ld_tag(p.gpart + tid);
            ok = tag_ok(w, ep);
            S.gsum[tid] = __uint_as_float((uint32_t)w);
          }
          return ok;
        }, 2, 1, false))
      return;
    if (tid < R) {
      float t = 0.f;
      for (int q = 0; q < NQ; ++q) t += S.gsum[tid * NQ + q];
      S.sgw[tid] = 1.f / (1.f + __expf(-t));
    }
    __syncthreads();
  }
  Window<1, FragD<F8>> w3;
  w3.prime(p3_next);
  TL(9);
  if (Is > 0 && !wait_cnt<false>(p, bk, &bk->shared[0], 16, 1, (uint32_t)n_sb, false, &S.flags[3], 2, ep, (uint32_t)D))
    return;
  if (hn == 0) return;
  {  // stage the shared a [R][Is] into LDS, plus its zero row
    const int ns8 = R * Is / 8;
    for (int base = 0; base < ns8; base += NT * 4) {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e8 = base + k * NT + tid;
        v[k] = ld16<CP_SC1>(rs_as, e8 < ns8 ? (uint32_t)e8 * 16u : OOB);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e8 = base + k * NT + tid;
        if (e8 < ns8) *(u32x4*)(asl + ((e8 * 8) / Is) * p.ss + (e8 * 8) % Is) = v[k];
      }
    }
    for (int c = tid * 8; c < p.ss; c += NT * 8) *(u32x4*)(asl + szero * p.ss + c) = (u32x4){0u, 0u, 0u, 0u};
    __syncthreads();
  }
  // shared down: waves split the Is/32 chunks (their first weight loads went out before top-k)
  if (Is > 0) {
    f32x4 acc[MAX_BLK], acc1[MAX_BLK];  // (wide: acc1 is the second tile of rows)
#pragma unroll
    for (int bl = 0; bl < MAX_BLK; ++bl) acc[bl] = acc1[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
    int cu = c0s;
    const int srow = (i16 < R ? i16 : szero) * p.ss + g * 8;
    const int srow1 = (16 + i16 < R ? 16 + i16 : szero) * p.ss + g * 8;
    if (!wse) ws.prime(sd_next);
    ws.run(CPs, sd_next, [&](const FragSD& f) {
      const u32x4 b = lds16(asl + (cu < Cs ? srow + cu * 32 : szero * p.ss));
#pragma unroll
      for (int bl = 0; bl < MAX_BLK; ++bl)
        if (bl < nblk) acc[bl] = mfma(as_bf16x8(f.a[bl]), as_bf16x8(b), acc[bl]);
      if constexpr (WIDE) {
        const u32x4 b1 = lds16(asl + (cu < Cs ? srow1 + cu * 32 : szero * p.ss));
#pragma unroll
        for (int bl = 0; bl < MAX_BLK; ++bl)
          if (bl < nblk) acc1[bl] = mfma(as_bf16x8(f.a[bl]), as_bf16x8(b1), acc1[bl]);
      }
      ++cu;
    });
#pragma unroll
    for (int bl = 0; bl < MAX_BLK; ++bl) {
      if (bl < nblk) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int hh = 16 * bl + 4 * g + qq;
          if (hh < hn && i16 < R) s_shp[(wave * R + i16) * HR + hh] = acc[bl][qq];
          if (WIDE && hh < hn && 16 + i16 < R) s_shp[(wave * R + 16 + i16) * HR + hh] = acc1[bl][qq];
        }
      }
    }
  }
  // routed down: it needs every slot's a, so it waits for all gate/up units
  if (!wait_cnt<true>(p, bk, &bk->routed[0][0], 16, NRC, (uint32_t)(D * (I / 8)), false, &S.flags[4], 3, ep, (uint32_t)D))
    return;
  TL(10);
  if constexpr (!WIDE) {
    {  // stage the routed a [P][I] into LDS, plus its zero row
      if (tid < P) {  // pick -> its product row: the slot's users in row order
        const int d = S.eslot[S.ids[tid]], r = tid / K;
        S.ci[tid] = (int16_t)(S.slot_off[d] + __popc((uint32_t)S.slot_mask[d] & ((1u << r) - 1u)));
      }
      const int nr8 = P * I / 8;
      for (int base = 0; base < nr8; base += NT * 4) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e8 = base + k * NT + tid;
          v[k] = ld16<CP_SC1>(rs_ar, e8 < nr8 ? (uint32_t)e8 * 16u : OOB);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e8 = base + k * NT + tid;
          if (e8 < nr8) *(u32x4*)(al + ((e8 * 8) / I) * p.as + (e8 * 8) % I) = v[k];
        }
      }
      for (int c = tid * 8; c < p.as; c += NT * 8) *(u32x4*)(al + azero * p.as + c) = (u32x4){0u, 0u, 0u, 0u};
      __syncthreads();
    }
    // routed down: slot d on wave d % NW; frags of up to 4 column groups (slot, part)
    {
      f32x4 acc[MAX_BLK];
#pragma unroll
      for (int bl = 0; bl < MAX_BLK; ++bl) acc[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
      int ju = 0, qu = 0;
      w3.run(nsl * NP3, p3_next, [&](const FragD<F8>& f) {
        const int d = wave + NW * ju;
        const int m = __popc((uint32_t)S.slot_mask[d]), ci0 = S.slot_off[d];
        const int arow = (i16 < m ? ci0 + i16 : azero) * p.as + g * 32;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int t3 = 2 * qu + t, c = 4 * t3 + g;
          if (t3 < TI) {
            u32x4 b[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) b[q] = lds16(al + (c < CI ? arow + t3 * 128 + 8 * q : azero * p.as));
#pragma unroll
            for (int bl = 0; bl < MAX_BLK; ++bl) {
              if (bl < nblk) {
                const uint32_t sb = f.s[bl][t] >> (8 * ((s3r + (16 * bl + i16) * CI + c) & 3));
                const float sc = e8m0f(sb & 0xFFu);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const bf16x8 aq = F8 ? fp8x8(f.a[t][(q >> 1) & (F8 ? 1 : 0)][bl][2 * (q & 1)],
                                               f.a[t][(q >> 1) & (F8 ? 1 : 0)][bl][2 * (q & 1) + 1], sc)
                                       : fp4x8(f.a[t][0][bl][q], sc);
                  acc[bl] = mfma(aq, as_bf16x8(b[q]), acc[bl]);
                }
              }
            }
          }
        }
        if (++qu == NP3) {
          qu = 0;
#pragma unroll
          for (int bl = 0; bl < MAX_BLK; ++bl) {
            if (bl < nblk) {
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) {
                const int hh = 16 * bl + 4 * g + qq;
                if (hh < hn && i16 < m) s_outp[(ci0 + i16) * HR + hh] = acc[bl][qq];
              }
            }
            acc[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
          ++ju;
        }
      });
    }
  } else {
    if (tid < P) {  // pick -> its product row: the expert's users in row order (wide)
      const int e = S.ids[tid], d = S.eslot[e], r = tid / K;
      S.ci[tid] = (int16_t)(S.slot_off[d] + __popc(S.rowmask[e] & ((1u << r) - 1u)));  // over the expert's slots
    }
    // stage product rows [pr0, pr0 + n) of the routed a into LDS rows [0, n)
    auto stage_a = [&](int pr0, int n) {
      const int nr8 = n * I / 8, b8 = pr0 * I / 8;
      for (int base = 0; base < nr8; base += NT * 4) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e8 = base + k * NT + tid;
          v[k] = ld16<CP_SC1>(rs_ar, e8 < nr8 ? (uint32_t)(b8 + e8) * 16u : OOB);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e8 = base + k * NT + tid;
          if (e8 < nr8) *(u32x4*)(al + ((e8 * 8) / I) * p.as + (e8 * 8) % I) = v[k];
        }
      }
    };
    // routed down: slot d on wave d % NW; frags of up to 4 column groups (slot, part)
    {
      f32x4 acc[MAX_BLK];
#pragma unroll
      for (int bl = 0; bl < MAX_BLK; ++bl) acc[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
      int ju = 0, qu = 0;
      int abase = 0;  // product row held in LDS row 0
      auto down_use = [&](const FragD<F8>& f) {
        const int d = wave + NW * ju;
        const int m = __popc((uint32_t)S.slot_mask[d]), ci0 = S.slot_off[d];
        const int arow = (i16 < m ? ci0 - abase + i16 : azero) * p.as + g * 32;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int t3 = 2 * qu + t, c = 4 * t3 + g;
          if (t3 < TI) {
            u32x4 b[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) b[q] = lds16(al + (c < CI ? arow + t3 * 128 + 8 * q : azero * p.as));
#pragma unroll
            for (int bl = 0; bl < MAX_BLK; ++bl) {
              if (bl < nblk) {
                const uint32_t sb = f.s[bl][t] >> (8 * ((s3r + (16 * bl + i16) * CI + c) & 3));
                const float sc = e8m0f(sb & 0xFFu);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const bf16x8 aq = F8 ? fp8x8(f.a[t][(q >> 1) & (F8 ? 1 : 0)][bl][2 * (q & 1)],
                                               f.a[t][(q >> 1) & (F8 ? 1 : 0)][bl][2 * (q & 1) + 1], sc)
                                       : fp4x8(f.a[t][0][bl][q], sc);
                  acc[bl] = mfma(aq, as_bf16x8(b[q]), acc[bl]);
                }
              }
            }
          }
        }
        if (++qu == NP3) {
          qu = 0;
#pragma unroll
          for (int bl = 0; bl < MAX_BLK; ++bl) {
            if (bl < nblk) {
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) {
                const int hh = 16 * bl + 4 * g + qq;
                if (hh < hn && i16 < m) s_outp[(ci0 + i16) * HR + hh] = acc[bl][qq];
              }
            }
            acc[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
          ++ju;
        }
      };
      // groups of consecutive slots whose product rows fit in the azero rows
      // of LDS (which overlap the shared a, no longer read); each wave's
      // window runs on across the groups: the frag in flight at a group's end
      // is the wave's first of the next group
      int ga = 0, jw = 0, used = 0;
      while (ga < D) {
        const int base = S.slot_off[ga];
        int lo = ga + 1, hi = D;  // the last slot boundary gb with slot_off[gb] - base <= azero
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (S.slot_off[mid] - base <= azero)
            lo = mid;
          else
            hi = mid - 1;
        }
        const int gb = lo;
        __syncthreads();  // the previous group's readers (or the shared down) are done with the rows
        if (ga == 0)
          for (int c = tid * 8; c < p.as; c += NT * 8) *(u32x4*)(al + azero * p.as + c) = (u32x4){0u, 0u, 0u, 0u};
        stage_a(base, S.slot_off[gb] - base);
        __syncthreads();
        const int nw = (gb > wave ? (gb - wave + NW - 1) / NW : 0) - jw;  // this wave's slots in [ga, gb)
        abase = base;
        if (used & 1)
          w3.template run_rot<1>(nw * NP3, p3_next, down_use);
        else
          w3.template run_rot<0>(nw * NP3, p3_next, down_use);
        used += nw * NP3;
        jw += nw;
        ga = gb;
      }
    }
  }
  TL(11);
  __syncthreads();
  // combine in a fixed order: picks in (row, k) order, then the shared part
  if constexpr (!WIDE) {
    if (tid < R * hn) {
      const int r = tid / hn, hh = tid % hn, h = h0 + hh;
      float yr = 0.f;
      for (int k = 0; k < K; ++k) yr += S.w[r * K + k] * s_outp[S.ci[r * K + k] * HR + hh];
      float ys = 0.f;
      if (Is > 0)
        for (int w = 0; w < NW; ++w) ys += s_shp[(w * R + r) * HR + hh];
      if (FEAT && p.sgate && Is > 0) ys *= S.sgw[r];
      const uint32_t hb = f2bf(bf2f(cx) + (p.res ? bf2f(cr) : 0.f));
      p.out[(size_t)r * H + h] = (uint16_t)f2bf(bf2f(hb) + (yr + ys));
      if (p.dbg_yr) p.dbg_yr[(size_t)r * H + h] = yr;
      if (p.dbg_ys) p.dbg_ys[(size_t)r * H + h] = ys;
    }
  } else {
    auto combine = [&](int qc, uint32_t xb, uint32_t rbv) {
      const int r = qc / hn, hh = qc % hn, h = h0 + hh;
      float yr = 0.f;
      for (int k = 0; k < K; ++k) yr += S.w[r * K + k] * s_outp[S.ci[r * K + k] * HR + hh];
      float ys = 0.f;
      if (Is > 0)
        for (int w = 0; w < NW; ++w) ys += s_shp[(w * R + r) * HR + hh];
      if (FEAT && p.sgate && Is > 0) ys *= S.sgw[r];
      const uint32_t hb = f2bf(bf2f(xb) + (p.res ? bf2f(rbv) : 0.f));
      p.out[(size_t)r * H + h] = (uint16_t)f2bf(bf2f(hb) + (yr + ys));
      if (p.dbg_yr) p.dbg_yr[(size_t)r * H + h] = yr;
      if (p.dbg_ys) p.dbg_ys[(size_t)r * H + h] = ys;
    };
    if (tid < R * hn) combine(tid, cx, cr);
    if (WIDE && tid + NT < R * hn) combine(tid + NT, cx2, cr2);
  }
  TL(12);
}

// Separate kernels rather than run-time branches, so that each launch's code
// is compact: activations staged in LDS, or read from global scratch (wide
// rows); router sums by the last chunk's workgroup, or by every reader.  The
// _f kernels add the optional steps (the shared expert's gate, group-limited
// routing).  A call runs its code once, front to back, so code it does not
// execute still costs instruction fetches: the plain kernels carry none of it.
#define MT_KERNEL(NAME, XL, RS, FEAT, F8, WIDE)                  \
  __global__ __launch_bounds__(NT, 1) void NAME(Params p) {      \
    __shared__ SharedT<WIDE> S;                                  \
    extern __shared__ __attribute__((aligned(16))) char s_dyn[]; \
    tail<XL, RS, FEAT, F8, WIDE>(p, S, s_dyn);                   \
  }
// Every kernel of the tail; the narrow ones (up to 16 rows) are defined in
// moe_tail.hip, the wide ones (17..32 rows) in moe_tail_wide.hip, so that the
// narrow kernels' code object does not change with the wide ones.
#define MT_KERNEL_DECL(NAME) __global__ void NAME(Params p);
MT_KERNEL_DECL(moe_tail_kernel_lds)
MT_KERNEL_DECL(moe_tail_kernel_lds_rs)
MT_KERNEL_DECL(moe_tail_kernel_gm)
MT_KERNEL_DECL(moe_tail_kernel_lds_f)
MT_KERNEL_DECL(moe_tail_kernel_lds_rs_f)
MT_KERNEL_DECL(moe_tail_kernel_gm_f)
MT_KERNEL_DECL(moe_tail_kernel_lds_8)
MT_KERNEL_DECL(moe_tail_kernel_lds_rs_8)
MT_KERNEL_DECL(moe_tail_kernel_gm_8)
MT_KERNEL_DECL(moe_tail_kernel_lds_f8)
MT_KERNEL_DECL(moe_tail_kernel_lds_rs_f8)
MT_KERNEL_DECL(moe_tail_kernel_gm_f8)
MT_KERNEL_DECL(moe_tail_kernel_gm_w)
MT_KERNEL_DECL(moe_tail_kernel_gm_wf)
MT_KERNEL_DECL(moe_tail_kernel_gm_w8)
MT_KERNEL_DECL(moe_tail_kernel_gm_wf8)
#undef MT_KERNEL_DECL

}  // namespace mt
