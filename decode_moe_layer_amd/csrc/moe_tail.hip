// Fused decode MoE layer tail for MI355X (gfx950): one persistent launch.
//
// Steps (one tensor-parallel rank's shard, 1..16 rows), after "[AMD]
// integrate kimi k3 monokernel" (sglang PR 43481), K2 commit text, sections
// Motivation and "Kernel Replacement":
//   norm    h = bf16(x + residual); xn = bf16(h * rstd * gamma)
//   router  logits = xn . Wr^T (fp32)
//   top-k   K rounds of a wave-wide maximum, exact ties to the lower expert id
//           ("glm53: Long-context indexer ...", PR 85 commit row 9)
//   dedup   each distinct expert of the step is one slot with its using rows;
//           its weights stream from HBM once (PR 85 commit rows 16 and 20)
//   gate/up per (slot, 8 intermediate indices): 16 MFMA rows (8 gate + 8 up)
//           against all using rows as MFMA columns; a = silu(g) * u
//   shared  the bf16 shared expert's gate/up the same way
//   down    per CTA a range of hidden rows: every slot's down tile and the
//           shared down tile, products kept per (pick, row) in LDS
//   combine y = sum over picks in slot order of w * d, plus the shared
//           output, in fp32 and a fixed order; out = bf16(h + y)
//           (chunk-ordered fp32 partials: "Split the Kimi3 AttnRes mix across
//           CTAs for decode rows", flare PR 11, design section)
//
// Cross-workgroup exchange goes through handle-owned scratch: counters in two
// banks selected by the call's epoch (an atomic ticket / grid size), so no
// reset is needed between calls or graph replays; every wait has a deadline
// and a shared abort word (K2 commit text, Motivation: each wait has a
// deadline, a failed wait stops the launch everywhere).
//
// GEMV tiles use v_mfma_f32_16x16x32_bf16: weights are the A operand (16
// rows), activations the B operand (up to 16 rows as columns).  MXFP4 codes
// are dequantised exactly to bf16 with v_cvt_scalef32_pk_bf16_fp4 (E2M1 x
// 2^(s-127) is exact in bf16 for the scales in range), so every product is
// exact and accumulation is fp32.  A lane's 16-byte weight load is one whole
// 32-element scale block (PR 85 commit row 18's 16-byte loads); weights are
// read once per call with nontemporal loads (commit row 21).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_tail.h"

namespace mt {

constexpr int NT = 512;      // threads per workgroup
constexpr int NW = NT / 64;  // waves per workgroup
constexpr int NQ = 16;       // norm slices per row
constexpr int MAX_R = 16;
constexpr int MAX_E = 512;
constexpr int MAX_K = 32;
constexpr int MAX_P = MAX_R * MAX_K;  // picks per call
constexpr int MAX_BLK = 4;            // 16-row down blocks per workgroup
constexpr int DEPTH = 4;              // loads in flight per wave in the streams

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Bank {
  uint32_t norm;
  uint32_t _p0[63];
  uint32_t router;
  uint32_t _p1[63];
  uint32_t shared;
  uint32_t _p2[63];
  uint32_t routed;
  uint32_t _p3[63];
  uint32_t abort_;
  uint32_t _p4[63];
};

struct Ctl {
  unsigned long long ticket;
  uint32_t _p0[62];
  uint32_t error;
  uint32_t _p1[63];
  Bank bank[2];
};

struct Params {
  int R, H, E, K, I, Is, scoring, G;
  int shp_off;  // floats of the per-pick product area in dynamic LDS
  double eps;
  unsigned long long deadline_ticks;
  uint32_t debug_flags;
  int debug_block;
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
  uint16_t* out;
  uint16_t* res_out;
  int32_t* topk_ids;
  float* topk_w;
  float* dbg_logits;
  float* dbg_yr;
  float* dbg_ys;
  Ctl* ctl;
  uint16_t* xn;
  float* logits;
  uint16_t* a_s;
  uint16_t* a_r;
};

// ------------------------------------------------------------------ helpers --

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *(const uint32_t*)p; }

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

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// monotone map of a float onto uint32 (larger float -> larger key); -0 == +0
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// index of the n-th set bit of m (n < popcount(m))
__device__ __forceinline__ int nth_bit(uint32_t m, int n) {
  for (int k = 0; k < n; ++k) m &= m - 1;
  return __ffs(m) - 1;
}

// Rolling window over n items: item i's loads are issued DEPTH items before
// it is consumed, so each wave keeps DEPTH loads in flight.
template <class LoadF, class UseF>
__device__ __forceinline__ void stream(int n, LoadF load, UseF use) {
  using Frag = decltype(load(0));
  if (n <= 0) return;
  Frag buf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) buf[j] = load(j < n ? j : n - 1);
  for (int base = 0; base < n; base += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int i = base + j;
      if (i < n) {
        Frag cur = buf[j];
        const int nx = i + DEPTH;
        buf[j] = load(nx < n ? nx : n - 1);
        use(cur, i);
      }
    }
  }
}

// -------------------------------------------------------- cross-CTA sync --

// Make this workgroup's global writes visible at agent scope, then add n to *c.
__device__ __forceinline__ void publish(uint32_t* c, uint32_t n) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0 && n) __hip_atomic_fetch_add(c, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-uniform wait for *c >= target with a deadline.  Returns false when
// the launch is aborted (this wait timed out, or another one did).
__device__ bool wait_ge(const Params& p, Bank* bk, uint32_t* c, uint32_t target, bool stall, uint32_t* s_flag) {
  if (threadIdx.x == 0) {
    uint32_t ok = 1;
    const unsigned long long t0 = wall_clock64();
    while (true) {
      const uint32_t v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v >= target && !stall) break;
      if (__hip_atomic_load(&bk->abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        ok = 0;
        break;
      }
      if (wall_clock64() - t0 > p.deadline_ticks) {
        __hip_atomic_store(&bk->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.ctl->error, (uint32_t)MOE_TAIL_ETIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *s_flag = ok;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// Workgroup-wide exclusive scan of one int per thread (threads >= n give 0).
__device__ int block_exscan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) base += s_tmp[w];
    tot += s_tmp[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

struct FragBF {
  u32x4 a, b;
};
struct FragFP4 {
  u32x4 a;
  uint32_t s;
  u32x4 b[4];
};
struct FragDown {
  u32x4 a[MAX_BLK];
  uint32_t s[MAX_BLK];
  u32x4 b[4];
};
struct FragSDown {
  u32x4 a[MAX_BLK];
  u32x4 b;
};

// ------------------------------------------------------------------ kernel --

__global__ __launch_bounds__(NT, 1) void moe_tail_kernel(Params p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cta = blockIdx.x;
  const int R = p.R, H = p.H, E = p.E, K = p.K, I = p.I, Is = p.Is, G = p.G;
  const int P = R * K;

  __shared__ uint32_t s_flags[8];
  __shared__ uint32_t s_ep;
  __shared__ double s_tmpd[NW];
  __shared__ int s_tmpi[NW];
  __shared__ int s_ids[MAX_P];
  __shared__ float s_w[MAX_P];
  __shared__ int s_ci[MAX_P];
  __shared__ int s_minpick[MAX_E];
  __shared__ uint32_t s_rowmask[MAX_E];
  __shared__ int s_eslot[MAX_E];
  __shared__ int s_slot_expert[MAX_P];
  __shared__ uint32_t s_slot_mask[MAX_P];
  __shared__ int s_slot_off[MAX_P + 1];
  __shared__ int s_nslot;
  __shared__ f32x4 s_red[2][NW][64];
  extern __shared__ float s_dyn[];

  // ---- epoch ticket: bank = ep & 1; workgroup 0 clears the next bank
  if (tid == 0) {
    const unsigned long long t = __hip_atomic_fetch_add(&p.ctl->ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ep = (uint32_t)(t / (unsigned long long)G);
  }
  __syncthreads();
  const uint32_t ep = s_ep;
  Bank* bk = &p.ctl->bank[ep & 1];
  if (cta == 0) {
    uint32_t* nb = (uint32_t*)&p.ctl->bank[(ep + 1) & 1];
    for (int i = tid; i < (int)(sizeof(Bank) / 4); i += NT) nb[i] = 0;
  }
  const bool stall = (p.debug_flags & MOE_TAIL_DEBUG_STALL) && cta == p.debug_block;

  // ---- P0: fused residual add + RMSNorm; workgroup c < R*NQ owns a slice
  if (cta < R * NQ) {
    const int row = cta / NQ, q = cta % NQ;
    const uint16_t* xr = p.x + (size_t)row * H;
    const uint16_t* rr = p.res ? p.res + (size_t)row * H : nullptr;
    double ss = 0.0;
    for (int i = tid * 8; i < H; i += NT * 8) {
      const u32x4 xv = ld16(xr + i);
      const u32x4 rv = rr ? ld16(rr + i) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double h0 = bf2f(f2bf(bf2f(xv[k] & 0xFFFFu) + bf2f(rv[k] & 0xFFFFu)));
        const double h1 = bf2f(f2bf(bf2f(xv[k] >> 16) + bf2f(rv[k] >> 16)));
        ss = fma(h0, h0, ss);
        ss = fma(h1, h1, ss);
      }
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) s_tmpd[wave] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int w = 0; w < NW; ++w) tot += s_tmpd[w];
    const double rstd = 1.0 / sqrt(tot / (double)H + p.eps);
    const int SL = H / NQ, s0 = q * SL;
    for (int i = s0 + tid * 8; i < s0 + SL; i += NT * 8) {
      const u32x4 xv = ld16(xr + i);
      const u32x4 rv = rr ? ld16(rr + i) : (u32x4){0u, 0u, 0u, 0u};
      const u32x4 gv = ld16(p.gamma + i);
      u32x4 hv, nv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h0 = f2bf(bf2f(xv[k] & 0xFFFFu) + bf2f(rv[k] & 0xFFFFu));
        const uint32_t h1 = f2bf(bf2f(xv[k] >> 16) + bf2f(rv[k] >> 16));
        const uint32_t n0 = d2bf(((double)bf2f(h0) * rstd) * (double)bf2f(gv[k] & 0xFFFFu));
        const uint32_t n1 = d2bf(((double)bf2f(h1) * rstd) * (double)bf2f(gv[k] >> 16));
        hv[k] = h0 | (h1 << 16);
        nv[k] = n0 | (n1 << 16);
      }
      *(u32x4*)(p.xn + (size_t)row * H + i) = nv;
      if (p.res_out) *(u32x4*)(p.res_out + (size_t)row * H + i) = hv;
    }
    publish(&bk->norm, 1);
  }
  if (!wait_ge(p, bk, &bk->norm, (uint32_t)(R * NQ), stall, &s_flags[0])) return;

  // ---- P1: router row blocks and shared gate/up blocks (waves split K)
  const int n_rb = (E + 15) / 16, n_sb = Is / 8, n_p1 = n_rb + n_sb;
  {
    const int T1 = H / 32, TP1 = (T1 + NW - 1) / NW;
    const int t0 = min(T1, wave * TP1), t1 = min(T1, t0 + TP1);
    const int i = lane & 15, g = lane >> 4, j = lane & 15;
    uint32_t nr = 0, ns = 0;
    for (int u = cta; u < n_p1; u += G) {
      const bool is_router = u < n_rb;
      const uint16_t* arow;
      bool avalid = true;
      if (is_router) {
        const int e = u * 16 + i;
        avalid = e < E;
        arow = p.rw + (size_t)(avalid ? e : E - 1) * H;
      } else {
        const int sb = u - n_rb;
        arow = p.ws13 + (size_t)(i < 8 ? sb * 8 + i : Is + sb * 8 + (i - 8)) * H;
      }
      const bool bvalid = j < R;
      const uint16_t* brow = p.xn + (size_t)(bvalid ? j : 0) * H;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      stream(
          t1 - t0,
          [&](int k) {
            const int t = t0 + k;
            FragBF f;
            f.a = avalid ? ld16_nt(arow + t * 32 + g * 8) : (u32x4){0u, 0u, 0u, 0u};
            f.b = bvalid ? ld16(brow + t * 32 + g * 8) : (u32x4){0u, 0u, 0u, 0u};
            return f;
          },
          [&](const FragBF& f, int) { acc = mfma(as_bf16x8(f.a), as_bf16x8(f.b), acc); });
      s_red[0][wave][lane] = acc;
      __syncthreads();
      if (is_router) {
        if (tid < 256) {
          const int l = tid >> 2, qq = tid & 3;
          float v = 0.f;
          for (int w = 0; w < NW; ++w) v += s_red[0][w][l][qq];
          const int e = u * 16 + 4 * (l >> 4) + qq, col = l & 15;
          if (e < E && col < R) p.logits[(size_t)col * E + e] = v;
        }
        ++nr;
      } else {
        if (tid < 128) {
          const int l = tid >> 2, qq = tid & 3;
          float gsum = 0.f, usum = 0.f;
          for (int w = 0; w < NW; ++w) {
            gsum += s_red[0][w][l][qq];
            usum += s_red[0][w][l + 32][qq];
          }
          const int ii = 4 * (l >> 4) + qq, col = l & 15;
          const float a = gsum / (1.f + __expf(-gsum)) * usum;
          if (col < R) p.a_s[(size_t)col * Is + (u - n_rb) * 8 + ii] = (uint16_t)f2bf(a);
        }
        ++ns;
      }
      __syncthreads();
    }
    if (nr) publish(&bk->router, nr);
    if (ns) publish(&bk->shared, ns);
  }

  // ---- top-k on every workgroup (identical inputs, identical result)
  if (!wait_ge(p, bk, &bk->router, (uint32_t)n_rb, false, &s_flags[1])) return;
  for (int r = wave; r < R; r += NW) {
    uint32_t key[8];
    float lg[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int e = lane + 64 * v;
      if (e < E) {
        const float l = p.logits[(size_t)r * E + e];
        lg[v] = l;
        const float kf = p.scoring == MOE_TAIL_SOFTMAX ? l : 1.f / (1.f + __expf(-l)) + p.bias[e];
        key[v] = ord_key(kf);
      } else {
        lg[v] = 0.f;
        key[v] = 0u;
      }
    }
    for (int k = 0; k < K; ++k) {
      uint32_t bkey = key[0];
      int bv = 0;
#pragma unroll
      for (int v = 1; v < 8; ++v)
        if (key[v] > bkey) {
          bkey = key[v];
          bv = v;
        }
      const uint32_t m = wave_max_u32(bkey);
      const unsigned long long bal = __ballot(bkey == m);
      int id;
      if (__popcll(bal) == 1) {
        id = __shfl(lane + 64 * bv, __ffsll((long long)bal) - 1);
      } else {
        id = wave_min_i32(bkey == m ? lane + 64 * bv : 0x7FFFFFFF);
      }
      float lsel = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v)
        if (lane == (id & 63) && v == (id >> 6)) {
          key[v] = 0u;
          lsel = lg[v];
        }
      lsel = __shfl(lsel, id & 63);
      if (lane == 0) {
        s_ids[r * K + k] = id;
        s_w[r * K + k] = lsel;
      }
    }
    // normalised weights over the K picks (lanes k < K)
    const float l0 = s_w[r * K];
    float t = 0.f;
    if (lane < K) {
      const float l = s_w[r * K + lane];
      t = p.scoring == MOE_TAIL_SOFTMAX ? __expf(l - l0) : 1.f / (1.f + __expf(-l));
    }
    const float sum = wave_sum_f32(t);
    if (lane < K) s_w[r * K + lane] = t / sum;
  }

  // ---- de-duplication: slot = distinct expert, in order of first pick
  for (int e = tid; e < E; e += NT) {
    s_minpick[e] = 0x7FFFFFFF;
    s_rowmask[e] = 0u;
  }
  __syncthreads();
  for (int q = tid; q < P; q += NT) {
    atomicMin(&s_minpick[s_ids[q]], q);
    atomicOr(&s_rowmask[s_ids[q]], 1u << (q / K));
  }
  __syncthreads();
  {
    const bool first = tid < P && s_minpick[s_ids[tid]] == tid;
    int nslot;
    const int slot = block_exscan(first ? 1 : 0, s_tmpi, &nslot);
    if (first) {
      const int e = s_ids[tid];
      s_eslot[e] = slot;
      s_slot_expert[slot] = e;
      s_slot_mask[slot] = s_rowmask[e];
    }
    if (tid == 0) s_nslot = nslot;
    __syncthreads();
    const int m = tid < nslot ? __popc(s_slot_mask[tid]) : 0;
    int tot;
    const int off = block_exscan(m, s_tmpi, &tot);
    if (tid < nslot) s_slot_off[tid] = off;
    if (tid == 0) s_slot_off[nslot] = tot;
    __syncthreads();
    if (tid < P) {
      const int e = s_ids[tid], d = s_eslot[e], r = tid / K;
      s_ci[tid] = s_slot_off[d] + __popc(s_slot_mask[d] & ((1u << r) - 1u));
    }
    __syncthreads();
  }
  const int D = s_nslot;
  if (cta == 0) {
    for (int q = tid; q < P; q += NT) {
      if (p.topk_ids) p.topk_ids[q] = s_ids[q];
      if (p.topk_w) p.topk_w[q] = s_w[q];
    }
    if (p.dbg_logits)
      for (int q = tid; q < R * E; q += NT) p.dbg_logits[q] = p.logits[q];
  }

  // ---- P2: routed gate/up units (slot, 8 intermediate indices)
  const int UB = I / 8, n_p2 = D * UB;
  {
    const int T2 = H / 128, TP2 = (T2 + NW - 1) / NW;
    const int t0 = min(T2, wave * TP2), t1 = min(T2, t0 + TP2);
    const int i = lane & 15, g = lane >> 4, j = lane & 15;
    const int off = n_p1 % G;
    uint32_t nu = 0;
    int buf = 0;
    for (int u = (cta - off + G) % G; u < n_p2; u += G, buf ^= 1) {
      const int d = u / UB, b = u % UB;
      const int e = s_slot_expert[d];
      const uint32_t mask = s_slot_mask[d];
      const int m = __popc(mask), ci0 = s_slot_off[d];
      const int wrow = i < 8 ? b * 8 + i : I + b * 8 + (i - 8);
      const uint8_t* arow = p.w13q + ((size_t)e * 2 * I + wrow) * (size_t)(H / 2);
      const uint8_t* srow = p.w13s + ((size_t)e * 2 * I + wrow) * (size_t)(H / 32);
      const bool bvalid = j < m;
      const uint16_t* brow = p.xn + (size_t)(bvalid ? nth_bit(mask, j) : 0) * H;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      stream(
          t1 - t0,
          [&](int k) {
            const int t = t0 + k, c = 4 * t + g;
            FragFP4 f;
            f.a = ld16_nt(arow + c * 16);
            f.s = ld4(srow + 4 * t);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              f.b[q] = bvalid ? ld16(brow + c * 32 + 8 * q) : (u32x4){0u, 0u, 0u, 0u};
            return f;
          },
          [&](const FragFP4& f, int) {
            const float sc = e8m0f((f.s >> (8 * g)) & 0xFFu);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = mfma(fp4x8(f.a[q], sc), as_bf16x8(f.b[q]), acc);
          });
      s_red[buf][wave][lane] = acc;
      __syncthreads();
      if (tid < 128) {
        const int l = tid >> 2, qq = tid & 3;
        float gsum = 0.f, usum = 0.f;
        for (int w = 0; w < NW; ++w) {
          gsum += s_red[buf][w][l][qq];
          usum += s_red[buf][w][l + 32][qq];
        }
        const int ii = 4 * (l >> 4) + qq, col = l & 15;
        const float a = gsum / (1.f + __expf(-gsum)) * usum;
        if (col < m) p.a_r[(size_t)(ci0 + col) * I + b * 8 + ii] = (uint16_t)f2bf(a);
      }
      ++nu;
    }
    if (nu) publish(&bk->routed, nu);
  }

  // ---- P3: down projections for this workgroup's hidden rows, then combine
  if (Is > 0 && !wait_ge(p, bk, &bk->shared, (uint32_t)n_sb, false, &s_flags[2])) return;
  if (!wait_ge(p, bk, &bk->routed, (uint32_t)n_p2, false, &s_flags[3])) return;
  const int HR = (H + G - 1) / G;
  const int h0 = cta * HR, hn = max(0, min(H, h0 + HR) - h0);
  if (hn == 0) return;
  const int nblk = (hn + 15) / 16;
  float* s_outp = s_dyn;                             // [P][HR]
  float* s_shp = s_dyn + p.shp_off;                  // [NW][R][HR]
  {
    const int i = lane & 15, g = lane >> 4, j = lane & 15;
    // shared down: waves split the Is/32 chunks
    if (Is > 0) {
      const int Cs = Is / 32, CP = (Cs + NW - 1) / NW;
      const int c0 = min(Cs, wave * CP), c1 = min(Cs, c0 + CP);
      const bool bvalid = j < R;
      f32x4 acc[MAX_BLK];
#pragma unroll
      for (int bl = 0; bl < MAX_BLK; ++bl) acc[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
      stream(
          c1 - c0,
          [&](int k) {
            const int c = c0 + k;
            FragSDown f;
#pragma unroll
            for (int bl = 0; bl < MAX_BLK; ++bl) {
              const int hh = 16 * bl + i;
              f.a[bl] = (bl < nblk && hh < hn) ? ld16_nt(p.ws2 + (size_t)(h0 + hh) * Is + c * 32 + g * 8)
                                               : (u32x4){0u, 0u, 0u, 0u};
            }
            f.b = bvalid ? ld16(p.a_s + (size_t)j * Is + c * 32 + g * 8) : (u32x4){0u, 0u, 0u, 0u};
            return f;
          },
          [&](const FragSDown& f, int) {
#pragma unroll
            for (int bl = 0; bl < MAX_BLK; ++bl)
              if (bl < nblk) acc[bl] = mfma(as_bf16x8(f.a[bl]), as_bf16x8(f.b), acc[bl]);
          });
#pragma unroll
      for (int bl = 0; bl < MAX_BLK; ++bl) {
        if (bl >= nblk) break;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int hh = 16 * bl + 4 * g + qq;
          if (hh < hn && j < R) s_shp[((size_t)wave * R + j) * HR + hh] = acc[bl][qq];
        }
      }
    }
    // routed down: slot d on wave d % NW; items (slot, t) with t over I/128
    const int CI = I / 32, TI = (CI + 3) / 4;
    const int nsl = D > wave ? (D - wave + NW - 1) / NW : 0;
    f32x4 acc[MAX_BLK];
#pragma unroll
    for (int bl = 0; bl < MAX_BLK; ++bl) acc[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
    stream(
        nsl * TI,
        [&](int k) {
          const int d = wave + NW * (k / TI), t = k % TI, c = 4 * t + g;
          const int e = s_slot_expert[d];
          const int m = __popc(s_slot_mask[d]), ci0 = s_slot_off[d];
          const bool cvalid = c < CI;
          FragDown f;
#pragma unroll
          for (int bl = 0; bl < MAX_BLK; ++bl) {
            const int hh = 16 * bl + i;
            const bool v = bl < nblk && hh < hn && cvalid;
            const size_t rowi = (size_t)e * H + (size_t)(h0 + (v ? hh : 0));
            f.a[bl] = v ? ld16_nt(p.w2q + rowi * (I / 2) + c * 16) : (u32x4){0u, 0u, 0u, 0u};
            f.s[bl] = v ? (uint32_t)p.w2s[rowi * CI + c] : 127u;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            f.b[q] = (j < m && cvalid) ? ld16(p.a_r + (size_t)(ci0 + j) * I + c * 32 + 8 * q) : (u32x4){0u, 0u, 0u, 0u};
          return f;
        },
        [&](const FragDown& f, int k) {
#pragma unroll
          for (int bl = 0; bl < MAX_BLK; ++bl) {
            if (bl < nblk) {
              const float sc = e8m0f(f.s[bl]);
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[bl] = mfma(fp4x8(f.a[bl][q], sc), as_bf16x8(f.b[q]), acc[bl]);
            }
          }
          if (k % TI == TI - 1) {
            const int d = wave + NW * (k / TI);
            const int m = __popc(s_slot_mask[d]), ci0 = s_slot_off[d];
#pragma unroll
            for (int bl = 0; bl < MAX_BLK; ++bl) {
              if (bl < nblk) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                  const int hh = 16 * bl + 4 * g + qq;
                  if (hh < hn && j < m) s_outp[(size_t)(ci0 + j) * HR + hh] = acc[bl][qq];
                }
              }
              acc[bl] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
          }
        });
  }
  __syncthreads();
  // combine in a fixed order: picks in (row, k) order, then the shared part
  for (int idx = tid; idx < R * hn; idx += NT) {
    const int r = idx / hn, hh = idx % hn, h = h0 + hh;
    float yr = 0.f;
    for (int k = 0; k < K; ++k) yr += s_w[r * K + k] * s_outp[(size_t)s_ci[r * K + k] * HR + hh];
    float ys = 0.f;
    if (Is > 0)
      for (int w = 0; w < NW; ++w) ys += s_shp[((size_t)w * R + r) * HR + hh];
    const uint32_t hb = f2bf(bf2f(p.x[(size_t)r * H + h]) + (p.res ? bf2f(p.res[(size_t)r * H + h]) : 0.f));
    p.out[(size_t)r * H + h] = (uint16_t)f2bf(bf2f(hb) + (yr + ys));
    if (p.dbg_yr) p.dbg_yr[(size_t)r * H + h] = yr;
    if (p.dbg_ys) p.dbg_ys[(size_t)r * H + h] = ys;
  }
}

}  // namespace mt

// ==================================================================== host ==

struct moe_tail {
  moe_tail_config cfg;
  int device;
  int G;
  size_t lds_dyn;
  unsigned long long deadline_ticks;
  void* scratch;
  mt::Ctl* ctl;
  uint16_t* xn;
  float* logits;
  uint16_t* a_s;
  uint16_t* a_r;
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

static size_t lds_dynamic_bytes(const moe_tail_config* c, int G) {
  const size_t HR = (size_t)(c->hidden + G - 1) / G;
  return ((size_t)c->max_rows * c->top_k * HR + (size_t)mt::NW * c->max_rows * HR) * sizeof(float);
}

extern "C" moe_tail_status moe_tail_check_config(const moe_tail_config* c) {
  if (!c) return fail(nullptr, MOE_TAIL_EINVAL, "config is NULL");
  if (c->max_rows < 1 || c->max_rows > mt::MAX_R)
    return fail(nullptr, MOE_TAIL_EINVAL, "max_rows %d outside 1..%d", c->max_rows, mt::MAX_R);
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
  if (c->debug_flags & ~MOE_TAIL_DEBUG_STALL) return fail(nullptr, MOE_TAIL_EINVAL, "unknown debug_flags bits");
  return MOE_TAIL_OK;
}

#define HIPCHK(h, call)                                                                       \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess) return fail((h), MOE_TAIL_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

extern "C" moe_tail_status moe_tail_create(const moe_tail_config* cfg, moe_tail_t** out) {
  if (!out) return fail(nullptr, MOE_TAIL_EINVAL, "out is NULL");
  *out = nullptr;
  moe_tail_status st = moe_tail_check_config(cfg);
  if (st != MOE_TAIL_OK) return st;
  int dev = cfg->device;
  if (dev < 0) HIPCHK(nullptr, hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIPCHK(nullptr, hipGetDeviceProperties(&prop, dev));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  const int G = prop.multiProcessorCount;
  const size_t dyn = lds_dynamic_bytes(cfg, G);
  hipFuncAttributes fa;
  HIPCHK(nullptr, hipFuncGetAttributes(&fa, (const void*)mt::moe_tail_kernel));
  if (dyn + fa.sharedSizeBytes > (size_t)prop.sharedMemPerBlock)
    return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "needs %zu B of LDS, device has %zu", dyn + fa.sharedSizeBytes,
                (size_t)prop.sharedMemPerBlock);
  if ((cfg->hidden + G - 1) / G > 16 * mt::MAX_BLK)
    return fail(nullptr, MOE_TAIL_EUNSUPPORTED, "hidden %d too large for %d workgroups", cfg->hidden, G);
  int wclk_khz = 0;
  HIPCHK(nullptr, hipDeviceGetAttribute(&wclk_khz, hipDeviceAttributeWallClockRate, dev));
  if (wclk_khz <= 0) wclk_khz = 100000;

  moe_tail_t* h = (moe_tail_t*)calloc(1, sizeof(moe_tail_t));
  if (!h) return fail(nullptr, MOE_TAIL_ENOMEM, "host allocation failed");
  h->cfg = *cfg;
  h->device = dev;
  h->G = G;
  h->lds_dyn = dyn;
  const unsigned long long us = cfg->deadline_us ? cfg->deadline_us : 200000u;
  h->deadline_ticks = us * (unsigned long long)wclk_khz / 1000ull;

  const size_t R = cfg->max_rows, H = cfg->hidden, E = cfg->num_experts, K = cfg->top_k;
  const size_t I = cfg->inter, Is = cfg->shared_inter;
  auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const size_t o_ctl = 0, o_xn = o_ctl + al(sizeof(mt::Ctl)), o_lg = o_xn + al(R * H * 2);
  const size_t o_as = o_lg + al(R * E * 4), o_ar = o_as + al(R * (Is ? Is : 1) * 2), total = o_ar + al(R * K * I * 2);
  int prev = 0;
  hipGetDevice(&prev);
  hipSetDevice(dev);
  hipError_t e = hipMalloc(&h->scratch, total);
  if (e != hipSuccess) {
    hipSetDevice(prev);
    free(h);
    return fail(nullptr, MOE_TAIL_ENOMEM, "hipMalloc(%zu): %s", total, hipGetErrorString(e));
  }
  e = hipMemset(h->scratch, 0, total);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)mt::moe_tail_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  hipSetDevice(prev);
  if (e != hipSuccess) {
    hipFree(h->scratch);
    free(h);
    return fail(nullptr, MOE_TAIL_EHIP, "scratch setup: %s", hipGetErrorString(e));
  }
  char* base = (char*)h->scratch;
  h->ctl = (mt::Ctl*)(base + o_ctl);
  h->xn = (uint16_t*)(base + o_xn);
  h->logits = (float*)(base + o_lg);
  h->a_s = (uint16_t*)(base + o_as);
  h->a_r = (uint16_t*)(base + o_ar);
  snprintf(h->err, sizeof(h->err), "no error");
  *out = h;
  return MOE_TAIL_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

extern "C" moe_tail_status moe_tail_run(moe_tail_t* h, int32_t rows, const moe_tail_args* a, void* stream) {
  if (!h) return fail(nullptr, MOE_TAIL_EINVAL, "handle is NULL");
  if (!a) return fail(h, MOE_TAIL_EINVAL, "args is NULL");
  const moe_tail_config& c = h->cfg;
  if (rows < 1 || rows > c.max_rows) return fail(h, MOE_TAIL_EINVAL, "rows %d outside 1..%d", rows, c.max_rows);
  const void* req[] = {a->x, a->gamma, a->router_w, a->w13_q, a->w13_s, a->w2_q, a->w2_s, a->out};
  const char* names[] = {"x", "gamma", "router_w", "w13_q", "w13_s", "w2_q", "w2_s", "out"};
  for (int k = 0; k < 8; ++k) {
    if (!req[k]) return fail(h, MOE_TAIL_EINVAL, "%s is NULL", names[k]);
    if (!aligned(req[k], 16)) return fail(h, MOE_TAIL_EINVAL, "%s is not 16-byte aligned", names[k]);
  }
  if (a->residual && !aligned(a->residual, 16)) return fail(h, MOE_TAIL_EINVAL, "residual is not 16-byte aligned");
  if (a->res_out && !aligned(a->res_out, 16)) return fail(h, MOE_TAIL_EINVAL, "res_out is not 16-byte aligned");
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
  p.G = h->G;
  p.shp_off = c.max_rows * c.top_k * ((c.hidden + h->G - 1) / h->G);
  p.eps = (double)c.eps;
  p.deadline_ticks = h->deadline_ticks;
  p.debug_flags = c.debug_flags;
  p.debug_block = c.debug_block;
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
  p.out = (uint16_t*)a->out;
  p.res_out = (uint16_t*)a->res_out;
  p.topk_ids = a->topk_ids;
  p.topk_w = a->topk_w;
  p.dbg_logits = a->dbg_logits;
  p.dbg_yr = a->dbg_y_routed;
  p.dbg_ys = a->dbg_y_shared;
  p.ctl = h->ctl;
  p.xn = h->xn;
  p.logits = h->logits;
  p.a_s = h->a_s;
  p.a_r = h->a_r;

  hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIPCHK(h, hipStreamIsCapturing(s, &cs));
  void* kargs[] = {&p};
  hipError_t e;
  if (cs == hipStreamCaptureStatusNone)
    e = hipLaunchCooperativeKernel((const void*)mt::moe_tail_kernel, dim3(h->G), dim3(mt::NT), kargs,
                                   (unsigned)h->lds_dyn, s);
  else
    e = hipLaunchKernel((const void*)mt::moe_tail_kernel, dim3(h->G), dim3(mt::NT), kargs, h->lds_dyn, s);
  if (e != hipSuccess) return fail(h, MOE_TAIL_EHIP, "kernel launch: %s", hipGetErrorString(e));
  return MOE_TAIL_OK;
}

extern "C" moe_tail_status moe_tail_get_error(moe_tail_t* h) {
  if (!h) return fail(nullptr, MOE_TAIL_EINVAL, "handle is NULL");
  uint32_t v = 0;
  int prev = 0;
  hipGetDevice(&prev);
  hipSetDevice(h->device);
  hipError_t e = hipMemcpy(&v, &h->ctl->error, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && v) e = hipMemset(&h->ctl->error, 0, 4);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  hipSetDevice(prev);
  if (e != hipSuccess) return fail(h, MOE_TAIL_EHIP, "reading the error word: %s", hipGetErrorString(e));
  if (v == MOE_TAIL_ETIMEOUT) return fail(h, MOE_TAIL_ETIMEOUT, "a cross-workgroup wait passed its deadline");
  return MOE_TAIL_OK;
}

extern "C" const char* moe_tail_strerror(moe_tail_t* h) { return h ? h->err : g_create_err; }

extern "C" void moe_tail_destroy(moe_tail_t* h) {
  if (!h) return;
  int prev = 0;
  hipGetDevice(&prev);
  hipSetDevice(h->device);
  hipFree(h->scratch);
  hipSetDevice(prev);
  free(h);
}
