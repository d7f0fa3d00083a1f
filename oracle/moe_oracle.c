/*
 * Plain CPU oracle of the decode MoE layer tail -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or helper with the HIP
 * path; it is written to be read against the pages and checked by eye.
 *
 * What it computes, per decode row, all in IEEE double precision:
 *   h      = bf16(x + r)                    fused residual add (rounded once)
 *   rstd   = 1 / sqrt(sum(h^2) / H + eps)
 *   xn     = bf16(h * rstd * gamma)         post-attention RMSNorm output
 *   l[e]   = sum_i xn[i] * Wr[e, i]         router logits (not rounded)
 *   key[e] = l[e]              (softmax scoring)
 *          = sigmoid(l[e]) + b[e]  (sigmoid scoring with a selection bias)
 *   S      = the K experts with the largest keys, ties to the lower id,
 *            listed by (key descending, id ascending)
 *            (group-limited: only experts of the topk_group groups whose two
 *            largest keys sum highest; see oracle_topk_grouped)
 *   w      = softmax(l[S])     (softmax scoring; equals p[S]/sum p[S])
 *          = sigmoid(l[S]) / sum sigmoid(l[S])   (sigmoid scoring)
 *            times the routed scaling factor (1 unless given)
 *   deq    = E2M1 x E8M0 (MXFP4) or E4M3 x E8M0 (MXFP8), blocks of 32
 *   for each pick e in S:  [g | u] = deq(W13[e]) xn,  a = g*sigmoid(g)*u,
 *                          d_e = deq(W2[e]) a
 *   s      = Ws2 (silu(Ws13_gate xn) * Ws13_up xn)   bf16 shared expert
 *   s      = sigmoid(wg . xn) s        only when a shared gate wg [H] is given
 *   folded norm (optional): the router and the shared gate/up project
 *            hg = bf16(h * gamma) instead of xn, and rstd multiplies their
 *            sums: l[e] = rstd * sum_i hg[i] Wr[e, i], likewise g and u of the
 *            shared expert; the routed experts and the gate still take xn
 *   y      = sum_k w_k d_{S_k} + s ;   out = bf16(h + y)
 *   front (optional, oracle_out_proj): x = bf16(attn . W_o^T), one rank's
 *            share of the attention output projection
 *
 * Sources (page titles; no listing is followed line by line):
 *   - "[AMD] integrate kimi k3 monokernel" (sglang PR 43481), K2 commit text,
 *     sections Motivation, Refusals and "Kernel Replacement": the tail's steps
 *     (fused add + RMSNorm, router GEMV, top-k with norm_topk_prob, MXFP4 routed
 *     experts gate/up + SiLU*up + down, bf16 shared expert, residual output).
 *   - "glm53: Long-context indexer ..." (sgl-amd-mono PR 86), PR 85 commit
 *     rows 9 and 20: top-k rounds that resolve exact ties toward the lower id.
 *   - the same K2 commit text, "Kernel Replacement": the shared expert's
 *     output is scaled by a sigmoid gate of the normed row
 *     (_fused_gate_sigmoid_mul_add_kernel); optional here.
 *   - "glm53: Long-context indexer ..." (sgl-amd-mono PR 86), PR 85's
 *     commit text (Motivation, and its commit on the router's norm): the
 *     router keeps bf16(a * gamma) with the sum of squares beside it, and the
 *     rstd then scales the logits and the activation blocks of the next
 *     projections (not bitwise equal to projecting the normed row).
 *   - OCP Microscaling Formats (MX) v1.0: E2M1 element and E8M0 scale
 *     encodings, blocks of 32 elements (the pages name MXFP4 but do not
 *     define it).
 * Readings where the pages are silent (gamma multiplies plainly, eps inside
 * the square root, gate rows first in W13, low nibble = even element; the
 * routed scaling factor, the shared-expert gate, group-limited routing,
 * MXFP8 codes and the folded norm as options that are off by default) are
 * listed with the design notes of the repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- number formats ------------------------------------------------------ */

/* E2M1 magnitudes, OCP MX v1.0 table for FP4: codes 0..7 (bit 3 is the sign). */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1(int code) {
  double m = kE2M1[code & 7];
  return (code & 8) ? -m : m;
}

/* E8M0: 2^(b-127); 0xFF encodes NaN. */
double oracle_e8m0(int b) {
  if ((b & 0xFF) == 0xFF) return NAN;
  return ldexp(1.0, (b & 0xFF) - 127);
}

/* E4M3 (OCP MX v1.0 FP8): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities. */
double oracle_e4m3(int code) {
  const int s = (code >> 7) & 1, e = (code >> 3) & 0xF, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

double oracle_dequant(int code, int scale_byte) {
  return oracle_e2m1(code) * oracle_e8m0(scale_byte);
}

double oracle_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to bfloat16, nearest with ties to even, from the exact value:
 * 8 significant bits for normals, quantum 2^-133 for subnormals, overflow to
 * infinity. */
uint16_t oracle_bf16_round(double v) {
  if (isnan(v)) return 0x7FC0;
  double a = fabs(v), q;
  if (a == 0.0) {
    q = 0.0;
  } else {
    int e;
    frexp(a, &e); /* a = m 2^e, 0.5 <= m < 1, so a in [2^(e-1), 2^e) */
    int qexp = e - 8; /* 8 significant bits */
    if (qexp < -133) qexp = -133;
    q = ldexp(nearbyint(ldexp(a, -qexp)), qexp); /* default rounding: to even */
  }
  float f = (float)q; /* exact: q has <= 8 significant bits */
  if (q >= ldexp(1.0, 128)) f = INFINITY;
  if (v < 0.0 || (v == 0.0 && signbit(v))) f = -f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* ---- the layer's steps --------------------------------------------------- */

static double bfd(const uint16_t* p, size_t i) { return oracle_bf16_to_double(p[i]); }

static double sigmoid(double t) { return 1.0 / (1.0 + exp(-t)); }

/* Fused residual add + RMSNorm of one row.  h_out, xn_out: [H] bf16 bits. */
void oracle_norm_row(int H, double eps, const uint16_t* x, const uint16_t* r, const uint16_t* gamma,
                     uint16_t* h_out, uint16_t* xn_out, double* rstd_out) {
  double ss = 0.0;
  for (int i = 0; i < H; i++) {
    double s = bfd(x, i) + (r ? bfd(r, i) : 0.0);
    h_out[i] = oracle_bf16_round(s);
    double h = bfd(h_out, i);
    ss += h * h;
  }
  double rstd = 1.0 / sqrt(ss / (double)H + eps);
  for (int i = 0; i < H; i++) xn_out[i] = oracle_bf16_round(bfd(h_out, i) * rstd * bfd(gamma, i));
  if (rstd_out) *rstd_out = rstd;
}

/* Router logits of one row: l[e] = sum_i xn[i] Wr[e,i]. */
void oracle_router_row(int H, int E, const uint16_t* xn, const uint16_t* router_w, double* logits) {
  for (int e = 0; e < E; e++) {
    double acc = 0.0;
    const uint16_t* w = router_w + (size_t)e * H;
    for (int i = 0; i < H; i++) acc += bfd(xn, i) * bfd(w, i);
    logits[e] = acc;
  }
}

/* Selection keys from logits. scoring 0: key = l; 1: key = sigmoid(l) + bias. */
void oracle_keys(int E, int scoring, const double* logits, const float* bias, double* keys) {
  for (int e = 0; e < E; e++) keys[e] = scoring == 0 ? logits[e] : sigmoid(logits[e]) + (double)bias[e];
}

/* Expert a beats expert b: larger key, or equal key and lower id. */
static int beats(const double* keys, int a, int b) {
  return keys[a] > keys[b] || (keys[a] == keys[b] && a < b);
}

/* Top-K by repeated selection of the best remaining expert. ids[0..K) in
 * (key descending, id ascending) order. */
void oracle_topk(int E, int K, const double* keys, int32_t* ids) {
  char* taken = (char*)calloc((size_t)E, 1);
  for (int k = 0; k < K; k++) {
    int best = -1;
    for (int e = 0; e < E; e++)
      if (!taken[e] && (best < 0 || beats(keys, e, best))) best = e;
    ids[k] = best;
    taken[best] = 1;
  }
  free(taken);
}

/* Normalised top-K weights. */
/* Group-limited top-K (parity unpinned with respect to the pages: the pages
 * do not describe group-limited routing; this rule is the build's own reading
 * of a routing variant, checked only against its own definition and special
 * cases).  The E experts form n_group groups of E / n_group
 * consecutive ids.  A group's score is the sum of its two largest keys (its
 * one key when a group has a single expert).  The topk_group groups with the
 * largest scores are kept (equal scores: the lower group first), and the
 * top-K of the kept experts follows, as oracle_topk orders it.  n_group <= 1
 * is oracle_topk itself.  K must not exceed topk_group * E / n_group. */
void oracle_topk_grouped(int E, int K, const double* keys, int n_group, int topk_group, int32_t* ids) {
  if (n_group <= 1) {
    oracle_topk(E, K, keys, ids);
    return;
  }
  const int gs = E / n_group;
  double* score = (double*)malloc(sizeof(double) * (size_t)n_group);
  char* kept = (char*)calloc((size_t)n_group, 1);
  char* taken = (char*)calloc((size_t)E, 1);
  for (int g = 0; g < n_group; g++) {
    double m1 = -INFINITY, m2 = -INFINITY;
    for (int e = g * gs; e < (g + 1) * gs; e++) {
      if (keys[e] > m1) {
        m2 = m1;
        m1 = keys[e];
      } else if (keys[e] > m2) {
        m2 = keys[e];
      }
    }
    score[g] = gs >= 2 ? m1 + m2 : m1;
  }
  for (int t = 0; t < topk_group; t++) {
    int best = -1;
    for (int g = 0; g < n_group; g++)
      if (!kept[g] && (best < 0 || score[g] > score[best])) best = g;
    kept[best] = 1;
  }
  for (int k = 0; k < K; k++) {
    int best = -1;
    for (int e = 0; e < E; e++)
      if (kept[e / gs] && !taken[e] && (best < 0 || beats(keys, e, best))) best = e;
    ids[k] = best;
    taken[best] = 1;
  }
  free(score);
  free(kept);
  free(taken);
}

void oracle_topk_weights(int K, int scoring, const double* logits, const int32_t* ids, double* w) {
  double sum = 0.0;
  if (scoring == 0) {
    double mx = -INFINITY;
    for (int k = 0; k < K; k++) mx = fmax(mx, logits[ids[k]]);
    for (int k = 0; k < K; k++) sum += (w[k] = exp(logits[ids[k]] - mx));
  } else {
    for (int k = 0; k < K; k++) sum += (w[k] = sigmoid(logits[ids[k]]));
  }
  for (int k = 0; k < K; k++) w[k] /= sum;
}

/* Dequantized element (row, col) of a [rows, cols] matrix with scales
 * [rows, cols/32].  MXFP4 (fmt 0): codes [rows, cols/2], low nibble = even
 * column.  MXFP8 (fmt 1): E4M3 codes [rows, cols], one byte per element. */
static double mx_at(int fmt, const uint8_t* q, const uint8_t* s, int cols, int row, int col) {
  const double sc = oracle_e8m0(s[(size_t)row * (cols / 32) + col / 32]);
  if (fmt == 1) return oracle_e4m3(q[(size_t)row * cols + col]) * sc;
  uint8_t byte = q[(size_t)row * (cols / 2) + col / 2];
  int code = (col & 1) ? (byte >> 4) : (byte & 0xF);
  return oracle_e2m1(code) * sc;
}

/* One routed expert on one row: d[H] = W2 (silu(g) * u), [g|u] = W13 xn. */
void oracle_expert_row(int fmt, int H, int I, const uint16_t* xn, const uint8_t* w13_q, const uint8_t* w13_s,
                       const uint8_t* w2_q, const uint8_t* w2_s, double* a_out, double* d_out) {
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  for (int i = 0; i < I; i++) {
    double g = 0.0, u = 0.0;
    for (int j = 0; j < H; j++) {
      double v = bfd(xn, j);
      g += mx_at(fmt, w13_q, w13_s, H, i, j) * v;
      u += mx_at(fmt, w13_q, w13_s, H, I + i, j) * v;
    }
    a[i] = g * sigmoid(g) * u;
    if (a_out) a_out[i] = a[i];
  }
  for (int h = 0; h < H; h++) {
    double acc = 0.0;
    for (int i = 0; i < I; i++) acc += mx_at(fmt, w2_q, w2_s, I, h, i) * a[i];
    d_out[h] = acc;
  }
  free(a);
}

/* The bf16 shared expert on one row: s[H].  Its gate and up sums are taken
 * over the activation row `act` and then multiplied by `scale` (1 for the
 * normed row xn; rstd for bf16(h * gamma) when the norm is folded). */
void oracle_shared_row_scaled(int H, int Is, const uint16_t* act, double scale, const uint16_t* ws13,
                              const uint16_t* ws2, double* s_out) {
  double* a = (double*)malloc(sizeof(double) * (size_t)Is);
  for (int i = 0; i < Is; i++) {
    double g = 0.0, u = 0.0;
    for (int j = 0; j < H; j++) {
      double v = bfd(act, j);
      g += bfd(ws13, (size_t)i * H + j) * v;
      u += bfd(ws13, (size_t)(Is + i) * H + j) * v;
    }
    g *= scale;
    u *= scale;
    a[i] = g * sigmoid(g) * u;
  }
  for (int h = 0; h < H; h++) {
    double acc = 0.0;
    for (int i = 0; i < Is; i++) acc += bfd(ws2, (size_t)h * Is + i) * a[i];
    s_out[h] = acc;
  }
  free(a);
}

void oracle_shared_row(int H, int Is, const uint16_t* xn, const uint16_t* ws13, const uint16_t* ws2,
                       double* s_out) {
  oracle_shared_row_scaled(H, Is, xn, 1.0, ws13, ws2, s_out);
}

/* bf16(h * gamma): the norm's input to the projections when rstd is folded
 * into their sums. */
static void folded_act(int H, const uint16_t* h, const uint16_t* gamma, uint16_t* hg) {
  for (int i = 0; i < H; i++) hg[i] = oracle_bf16_round(bfd(h, i) * bfd(gamma, i));
}

/* The shared expert's gate: sigmoid(wg . xn), the dot product in double. */
double oracle_shared_gate(int H, const uint16_t* xn, const uint16_t* wg) {
  double g = 0.0;
  for (int j = 0; j < H; j++) g += bfd(wg, j) * bfd(xn, j);
  return sigmoid(g);
}

/* The whole tail for `rows` rows.  Every output pointer may be NULL except
 * out.  Shapes: x, r, h_out, xn_out, out: [rows, H] bf16 bits; logits, keys:
 * [rows, E]; ids, w: [rows, K]; y_routed, y_shared: [rows, H].  sgate [H]
 * may be NULL (no shared gate); y_shared is the gated shared output. */
int oracle_moe_tail(int rows, int H, int E, int K, int I, int Is, int scoring, double eps, int n_group,
                    int topk_group, double routed_scale, int wfmt, int fold,
                    const uint16_t* x, const uint16_t* r, const uint16_t* gamma, const uint16_t* router_w,
                    const float* bias, const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                    const uint8_t* w2_s, const uint16_t* ws13, const uint16_t* ws2, const uint16_t* sgate,
                    uint16_t* h_out,
                    uint16_t* xn_out, double* logits_out, double* keys_out, int32_t* ids_out, double* w_out,
                    double* y_routed_out, double* y_shared_out, uint16_t* out) {
  if (rows < 0 || H <= 0 || H % 32 || E <= 0 || K <= 0 || K > E || I <= 0 || I % 32 || Is < 0 || !out) return 1;
  if (scoring == 1 && !bias) return 1;
  if (wfmt != 0 && wfmt != 1) return 1;
  if (n_group > 1 && (E % n_group || topk_group < 1 || topk_group > n_group || K > topk_group * (E / n_group)))
    return 1;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* xn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* hg = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  double* lg = (double*)malloc(sizeof(double) * (size_t)E);
  double* ky = (double*)malloc(sizeof(double) * (size_t)E);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  double* w = (double*)malloc(sizeof(double) * (size_t)K);
  double* d = (double*)malloc(sizeof(double) * (size_t)H);
  double* yr = (double*)malloc(sizeof(double) * (size_t)H);
  double* ys = (double*)malloc(sizeof(double) * (size_t)H);
  const size_t e13 = (size_t)2 * I * (wfmt == 1 ? H : H / 2), e13s = (size_t)2 * I * (H / 32);
  const size_t e2 = (size_t)H * (wfmt == 1 ? I : I / 2), e2s = (size_t)H * (I / 32);
  for (int row = 0; row < rows; row++) {
    const size_t ro = (size_t)row * H;
    double rstd;
    oracle_norm_row(H, eps, x + ro, r ? r + ro : NULL, gamma, h, xn, &rstd);
    if (fold) {
      folded_act(H, h, gamma, hg);
      oracle_router_row(H, E, hg, router_w, lg);
      for (int e = 0; e < E; e++) lg[e] *= rstd;
    } else {
      oracle_router_row(H, E, xn, router_w, lg);
    }
    oracle_keys(E, scoring, lg, bias, ky);
    oracle_topk_grouped(E, K, ky, n_group, topk_group, ids);
    oracle_topk_weights(K, scoring, lg, ids, w);
    for (int k = 0; k < K; k++) w[k] *= routed_scale;
    for (int j = 0; j < H; j++) yr[j] = 0.0;
    for (int k = 0; k < K; k++) {
      const int e = ids[k];
      oracle_expert_row(wfmt, H, I, xn, w13_q + e * e13, w13_s + e * e13s, w2_q + e * e2, w2_s + e * e2s, NULL, d);
      for (int j = 0; j < H; j++) yr[j] += w[k] * d[j];
    }
    for (int j = 0; j < H; j++) ys[j] = 0.0;
    if (Is > 0) oracle_shared_row_scaled(H, Is, fold ? hg : xn, fold ? rstd : 1.0, ws13, ws2, ys);
    if (Is > 0 && sgate) {
      const double sg = oracle_shared_gate(H, xn, sgate);
      for (int j = 0; j < H; j++) ys[j] *= sg;
    }
    for (int j = 0; j < H; j++) out[ro + j] = oracle_bf16_round(bfd(h, j) + (yr[j] + ys[j]));
    if (h_out) memcpy(h_out + ro, h, sizeof(uint16_t) * (size_t)H);
    if (xn_out) memcpy(xn_out + ro, xn, sizeof(uint16_t) * (size_t)H);
    if (logits_out) memcpy(logits_out + (size_t)row * E, lg, sizeof(double) * (size_t)E);
    if (keys_out) memcpy(keys_out + (size_t)row * E, ky, sizeof(double) * (size_t)E);
    if (ids_out) memcpy(ids_out + (size_t)row * K, ids, sizeof(int32_t) * (size_t)K);
    if (w_out) memcpy(w_out + (size_t)row * K, w, sizeof(double) * (size_t)K);
    if (y_routed_out) memcpy(y_routed_out + ro, yr, sizeof(double) * (size_t)H);
    if (y_shared_out) memcpy(y_shared_out + ro, ys, sizeof(double) * (size_t)H);
  }
  free(h); free(xn); free(hg); free(lg); free(ky); free(ids); free(w); free(d); free(yr); free(ys);
  return 0;
}

/* The out_proj in front of the tail, on one tensor-parallel rank's share
 * ("[AMD] integrate kimi k3 monokernel", K2 commit text, Motivation and
 * Modifications: the fused launch starts with the attention output
 * projection, whose result is all-reduced over the ranks before the norm).
 * attn [rows, A] bf16 is this rank's slice of the attention output and w_o
 * [H, A] bf16 the matching columns of the projection: y = attn . w_o^T in
 * double, and x = bf16(y) is the tail's input row.  On one GPU the rank's
 * partial stands for the all-reduced sum (the reduce itself is not run).
 * y_out may be NULL. */
void oracle_out_proj(int rows, int A, int H, const uint16_t* attn, const uint16_t* w_o, double* y_out,
                     uint16_t* x_out) {
  for (int r = 0; r < rows; r++)
    for (int h = 0; h < H; h++) {
      double acc = 0.0;
      for (int a = 0; a < A; a++) acc += bfd(attn, (size_t)r * A + a) * bfd(w_o, (size_t)h * A + a);
      if (y_out) y_out[(size_t)r * H + h] = acc;
      x_out[(size_t)r * H + h] = oracle_bf16_round(acc);
    }
}

/* Norm + router + keys only (used to check the top-k gap of generated rows). */
int oracle_router_keys(int rows, int H, int E, int scoring, double eps, int fold, const uint16_t* x,
                       const uint16_t* r, const uint16_t* gamma, const uint16_t* router_w, const float* bias,
                       double* logits_out, double* keys_out) {
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* xn = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  uint16_t* hg = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)H);
  for (int row = 0; row < rows; row++) {
    const size_t ro = (size_t)row * H;
    double* lg = logits_out + (size_t)row * E;
    double rstd;
    oracle_norm_row(H, eps, x + ro, r ? r + ro : NULL, gamma, h, xn, &rstd);
    if (fold) {
      folded_act(H, h, gamma, hg);
      oracle_router_row(H, E, hg, router_w, lg);
      for (int e = 0; e < E; e++) lg[e] *= rstd;
    } else {
      oracle_router_row(H, E, xn, router_w, lg);
    }
    oracle_keys(E, scoring, lg, bias, keys_out + (size_t)row * E);
  }
  free(h); free(xn); free(hg);
  return 0;
}
