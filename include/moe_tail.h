/*
 * moe_tail.h -- C ABI of the fused decode MoE layer tail for MI355X (gfx950).
 *
 * One call runs, for 1..16 decode rows of one tensor-parallel rank's shard,
 * in a single persistent HIP launch:
 *
 *   h       = bf16(x + residual)                      fused residual add
 *   xn      = bf16(h * rstd * gamma),  rstd = 1/sqrt(mean(h^2) + eps)
 *   logits  = xn . router_w^T                          (fp32, not rounded)
 *   top-k   softmax scoring: the K largest logits; weights = softmax over them
 *           sigmoid scoring: the K largest sigmoid(logit) + bias; weights =
 *           sigmoid(logit) / sum over the K picks (the bias selects only)
 *           ties always go to the lower expert id
 *   routed  for each pick e: a = silu(W13_gate[e] xn) * (W13_up[e] xn),
 *           d_e = W2[e] a, with MXFP4 weights (E2M1 codes, E8M0 block-32 scales)
 *   shared  s = Ws2 (silu(Ws13_gate xn) * (Ws13_up xn)), bf16 weights
 *   out     = bf16(h + sum_k w_k d_{e_k} + s),  res_out = h
 *
 * Sources: "[AMD] integrate kimi k3 monokernel" (sglang PR 43481), K2 commit
 * text, sections Motivation, Refusals and "Kernel Replacement" (the steps of
 * the tail and its refusals); "glm53: Long-context indexer ..." (sgl-amd-mono
 * PR 86), PR 85 commit table rows 9, 16, 18, 20, 21 (tie rule, expert
 * de-duplication, 16-byte and nontemporal weight loads); "Split the Kimi3
 * AttnRes mix across CTAs for decode rows" (flare PR 11), design section
 * (chunk-ordered fp32 partial sums, per-call tags); OCP Microscaling v1.0
 * (MXFP4 encoding).  There is no all-reduce: the result is one rank's
 * partial sum added to h.
 *
 * Conventions.  Every tensor pointer is a device pointer to caller-owned,
 * row-major, contiguous memory, 16-byte aligned.  The library reads the
 * weights in place and never copies them.  bf16 tensors are passed as raw
 * 16-bit patterns (void*).  No function throws; all report a status.
 */
#ifndef MOE_TAIL_H
#define MOE_TAIL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_tail moe_tail_t; /* opaque handle */

typedef enum {
  MOE_TAIL_OK = 0,
  MOE_TAIL_EINVAL = 1,        /* bad argument: size, pointer, alignment, rows */
  MOE_TAIL_EUNSUPPORTED = 2,  /* device is not gfx950, or limits exceeded */
  MOE_TAIL_ENOMEM = 3,        /* scratch allocation failed */
  MOE_TAIL_EHIP = 4,          /* a HIP runtime call failed */
  MOE_TAIL_ETIMEOUT = 5       /* a cross-workgroup wait passed its deadline */
} moe_tail_status;

typedef enum { MOE_TAIL_SOFTMAX = 0, MOE_TAIL_SIGMOID_BIAS = 1 } moe_tail_scoring;

/* Routed expert weight formats (OCP Microscaling Formats v1.0), both with one
 * E8M0 scale per 32 elements along K: MXFP4 packs two E2M1 codes per byte
 * (w13_q [E, 2I, H/2], w2_q [E, H, I/2]); MXFP8 has one E4M3 code per byte
 * (w13_q [E, 2I, H], w2_q [E, H, I]). */
typedef enum { MOE_TAIL_MXFP4 = 0, MOE_TAIL_MXFP8 = 1 } moe_tail_weight_format;

/* debug_flags bit: the workgroup `debug_block` never proceeds past its first
 * cross-workgroup wait until that wait's deadline fires (fault drill). */
#define MOE_TAIL_DEBUG_STALL 1u
/* debug_flags bit: the same, on the handle's first call only; later calls
 * run normally (drill of the recovery on one handle). */
#define MOE_TAIL_DEBUG_STALL_ONCE 2u

typedef struct {
  int32_t max_rows;     /* largest `rows` any run will pass: 1..32 (above 16, see moe_tail_run) */
  int32_t hidden;       /* H: multiple of 128, 128..16384 (a routed gate/up load step covers 128 columns of a
                           row: four 32-element scale blocks, one 16-byte load per lane; a norm slice is
                           H/16 columns in 8-element vectors); moe_tail_create also refuses (EUNSUPPORTED)
                           more than 32 hidden columns per compute unit, i.e. H > 8192 on a 256-CU device */
  int32_t num_experts;  /* E: 1..512 */
  int32_t top_k;        /* K: 1..min(E, 32) */
  int32_t inter;        /* I, per-rank expert intermediate: multiple of 32, 32..4096 */
  int32_t shared_inter; /* Is, per-rank shared intermediate: 0 (none) or multiple of 32, <= 4096 */
  int32_t scoring;      /* moe_tail_scoring */
  float eps;            /* RMSNorm epsilon, > 0 */
  int32_t device;       /* HIP device ordinal, or -1 for the current device */
  uint32_t deadline_us; /* per-wait deadline in microseconds; 0 selects 200000 */
  uint32_t debug_flags; /* 0 in production; see MOE_TAIL_DEBUG_STALL(_ONCE) */
  int32_t debug_block;  /* workgroup index used by debug_flags */
  /* routing variants, after the earlier fields so that zeroed configs keep
   * the plain routing: */
  int32_t n_group;      /* group-limited routing: groups of E / n_group consecutive experts (a multiple
                           of 8); a group scores the sum of its two largest selection keys, the
                           topk_group best groups are kept (equal scores: the lower group) and the
                           top-k is taken among their experts.  0 or 1: no groups */
  int32_t topk_group;   /* groups kept, 1..n_group, with K <= topk_group * E / n_group */
  float routed_scale;   /* routed scaling factor on the top-k weights; 0 means 1 */
  int32_t weight_format; /* routed expert codes: MOE_TAIL_MXFP4 (0) or MOE_TAIL_MXFP8 (1) */
  int32_t fold_norm;     /* 1: the norm is folded into the router and shared gate/up sums: they project
                            bf16(h * gamma) and are multiplied by the row's rstd afterwards ("glm53:
                            Long-context indexer ...", PR 85 commit text: the router's norm moves into its
                            logits; not bitwise equal to projecting xn).  The routed experts and the shared
                            gate still take xn.  0: plain (the router and shared expert project xn) */
  int32_t attn_dim;      /* A of the out_proj front: 0 (none), or a multiple of 128 up to 16384.  With A > 0
                            a call may pass attention rows instead of x (see moe_tail_args.attn) */
  int32_t w13_layout;    /* MXFP4 w13_q layout: 0 row-major [E, 2I, H/2]; 1 unit-blocked, in which the
                            codes a wave loads at once are contiguous: for expert e, unit b (intermediate
                            indices 8b..8b+7), column group c (elements 128c..128c+127) and lane
                            l = 16 q + i (q < 4, i < 16), bytes ((b H/128 + c) 64 + l) 16 .. +15 hold bytes
                            16q .. 16q+15 of column group c of row 8b + i (i < 8, gate) or I + 8b + i - 8
                            (up).  Same size as row-major; scales keep their layout */
} moe_tail_config;

typedef struct {
  /* inputs */
  const void* x;            /* [rows, H] bf16 post-attention activations */
  const void* residual;     /* [rows, H] bf16, or NULL (then h = x) */
  const void* gamma;        /* [H] bf16 RMSNorm weight */
  const void* router_w;     /* [E, H] bf16 */
  const float* router_bias; /* [E] fp32, required for MOE_TAIL_SIGMOID_BIAS, else ignored */
  const uint8_t* w13_q;     /* MXFP4 [E, 2I, H/2]: rows [0,I) gate, [I,2I) up; byte j = elements 2j (low nibble),
                               2j+1 (high).  MXFP8 [E, 2I, H]: byte j = element j */
  const uint8_t* w13_s;     /* [E, 2I, H/32] E8M0 scale of each 32-element block along H */
  const uint8_t* w2_q;      /* down projection codes: MXFP4 [E, H, I/2], same nibble order; MXFP8 [E, H, I] */
  const uint8_t* w2_s;      /* [E, H, I/32] E8M0 scales along I */
  const void* ws13;         /* [2Is, H] bf16 shared gate (rows [0,Is)) and up; NULL iff Is == 0 */
  const void* ws2;          /* [H, Is] bf16 shared down; NULL iff Is == 0 */
  /* outputs */
  void* out;                /* [rows, H] bf16: h + routed + shared */
  void* res_out;            /* [rows, H] bf16: h, or NULL */
  int32_t* topk_ids;        /* [rows, K] selected experts, (key desc, id asc) order, or NULL */
  float* topk_w;            /* [rows, K] normalised weights, or NULL */
  float* dbg_logits;        /* [rows, E] router logits, or NULL */
  float* dbg_y_routed;      /* [rows, H] fp32 routed sum, or NULL */
  float* dbg_y_shared;      /* [rows, H] fp32 shared expert output (after its gate), or NULL */
  /* optional input, after the outputs so that earlier callers' layouts hold */
  const void* shared_gate;  /* [H] bf16 gate wg, 16-byte aligned, or NULL: the shared output is
                               scaled by sigmoid(wg . xn) per row ("[AMD] integrate kimi k3
                               monokernel", K2 commit text, Kernel Replacement: the fused
                               gate-sigmoid-mul-add on the shared expert); ignored when Is == 0 */
  /* the out_proj front ("[AMD] integrate kimi k3 monokernel", K2 commit text, Motivation and
     Modifications: the fused launch starts with the attention output projection).  When attn is
     given, x must be NULL: the same launch computes x = bf16(attn . w_o^T) per row, each element
     summed in double and rounded once (every workgroup its own slice of the hidden columns), and
     the tail continues on that x.  One rank's share: on one GPU its partial stands for the
     all-reduced sum. */
  const void* attn;         /* [rows, A] bf16 attention output rows (this rank's slice), or NULL */
  const void* w_o;          /* [H, A] bf16 out_proj columns of this rank, required with attn */
} moe_tail_args;

/* Validate a configuration on the host only (no GPU call).  Returns
 * MOE_TAIL_OK or MOE_TAIL_EINVAL, with the reason in moe_tail_strerror(NULL).
 * The pages' fused tail refuses unsupported configurations at start-up rather
 * than falling back ("[AMD] integrate kimi k3 monokernel", K2 commit text,
 * section Refusals).  Limits that depend on the device (the compute-unit
 * count bounds H, LDS bounds rows x H) are checked only by moe_tail_create, so
 * an OK here is necessary, not sufficient: create's answer is final.
 * cfg is read and not kept. */
moe_tail_status moe_tail_check_config(const moe_tail_config* cfg);

/* Create a handle: validates cfg, checks the device is gfx950 and that one
 * workgroup of the persistent kernel fits on every compute unit (all of them
 * must be resident at once), allocates the handle-owned scratch (exchange
 * buffers, counters, error word) sized for max_rows, and zeroes it.  The
 * handle owns that scratch; the caller's tensors are never copied.  On
 * failure *out is NULL and moe_tail_strerror(NULL) holds the reason:
 * EINVAL (cfg), EUNSUPPORTED (not gfx950; H or LDS beyond this device),
 * ENOMEM, EHIP.  Source: "[AMD] integrate kimi k3 monokernel", K2 commit text,
 * section Modifications (one scratch buffer for each width; the launch reads
 * the serving engine's weights in place and makes no weight copies). */
moe_tail_status moe_tail_create(const moe_tail_config* cfg, moe_tail_t** out);

/* Enqueue one call on `stream` (a hipStream_t; NULL = default stream) and
 * return without synchronising.  The call is the whole tail in one persistent
 * launch ("[AMD] integrate kimi k3 monokernel", K2 commit text, Motivation:
 * the layer tail as a single launch; Kernel checks: graph replays of mixed
 * widths give the eager bits).  1 <= rows <= max_rows.  Up to 16 rows run
 * as a narrow launch (one 16-column MFMA tile of rows).  More rows (MTP
 * verify batches; the pages' launch falls back above concurrency 16, K2
 * commit text, section Speed) run as one wide launch when the handle allows
 * it: max_rows * top_k <= 512, attn_dim == 0 and its LDS plan fits the
 * device.  A wide launch de-duplicates experts across all rows, so each
 * distinct expert streams once per call; where rows are MFMA columns (router
 * and shared gate/up, shared down) a weight load feeds two 16-column tiles,
 * and an expert picked by more than 16 rows runs as one slot per 16 of them
 * (its weights are read once per slot).  A handle whose 16-row narrow
 * launch does not fit in LDS (many picks per row) runs every call as a wide
 * launch.  Otherwise calls above 16 rows run as ceil(rows / 16) narrow
 * launches over balanced row ranges, in order on the stream, each streaming
 * its own experts.  A row's outputs are the same bits at every width.
 * Graph-capturable:
 * the handle's per-call epoch lives in device memory, so replays need no
 * host work.  Calls on one handle must be ordered (one stream at a time).
 * Argument errors are returned synchronously and nothing is enqueued; a
 * device-side deadline is reported later by moe_tail_get_error. */
moe_tail_status moe_tail_run(moe_tail_t* h, int32_t rows, const moe_tail_args* args, void* stream);

/* Read and clear the sticky device error word (MOE_TAIL_OK or
 * MOE_TAIL_ETIMEOUT).  Every cross-workgroup wait has a deadline, and a wait
 * that passes it stops the whole launch ("[AMD] integrate kimi k3 monokernel",
 * K2 commit text, Motivation, and the fault row of Kernel checks).  Synchronises the device first.  While the word is set,
 * later calls on the handle give up at their first wait that is not already
 * satisfied (their outputs are then undefined); reading an error also resets
 * the handle's call epochs and counters, so the next call starts clean. */
moe_tail_status moe_tail_get_error(moe_tail_t* h);

/* Text of the last error reported on this handle (or on creation when h is
 * NULL); valid until the next call on the handle. */
const char* moe_tail_strerror(moe_tail_t* h);

/* Free the handle and its scratch.  The caller makes sure no run on it is
 * still in flight. */
void moe_tail_destroy(moe_tail_t* h);

/* Scratch bytes available to moe_tail_run_noalloc (4 MiB): enough for every
 * configuration up to 16 rows per launch with H <= 8192, E <= 512, K <= 10,
 * I <= 256 and Is <= 512 (at most 3.3 MB); larger ones are refused.  Where a
 * wide launch's scratch (more than 16 rows) does not fit, calls above 16 rows
 * run as narrow launches instead. */
#define MOE_TAIL_NOALLOC_SCRATCH_BYTES (4u << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Enqueues
 * one call like moe_tail_run, without a handle: the call's scratch (exchange
 * buffers, counters, epochs, error word) is a file-scope device array of
 * MOE_TAIL_NOALLOC_SCRATCH_BYTES on the current device, kept for the life of
 * the process; nothing is allocated, on the device or the host, and nothing
 * is copied.  cfg is validated as by moe_tail_create (device must be -1 or
 * the current device; MOE_TAIL_DEBUG_STALL_ONCE is refused), the other
 * arguments as by moe_tail_run; a configuration whose scratch would exceed
 * the array is refused with MOE_TAIL_EINVAL.  Errors are returned
 * synchronously, with the text in moe_tail_strerror(NULL).  The first call on
 * a device looks up the array's address on that device, once.
 *
 * Every call on a device shares that device's array and leaves its contents
 * for the next one (each call's words are tagged with per-workgroup call
 * counts that only grow, and each call clears the counters of the next), so
 * successive calls may change the configuration, the rows and the pointers.
 * Calls on one device must be ordered (one stream at a time): calls that
 * overlap on a device race on the array, with each other and with nothing
 * else (handles have scratch of their own).  A device-side deadline aborts
 * that call only (its outputs are undefined) and is not reported: the next
 * call starts clean.  Callers that need the report use a handle. */
moe_tail_status moe_tail_run_noalloc(const moe_tail_config* cfg, int32_t rows, const moe_tail_args* args,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TAIL_H */
