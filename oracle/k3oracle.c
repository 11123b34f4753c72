/*
 * k3oracle — plain fp64 CPU reference of the MXFP4 routed-expert path.
 *
 * TEST INFRASTRUCTURE ONLY: called by tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product path. Shares no code
 * with the GPU library. Written for clarity, not speed: every loop is the
 * definition it implements, in the order the pages give.
 *
 * Page abbreviations as in k3oracle.h: [A176], [SAT], [ZOR].
 */
#include "k3oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int g_threads = 1;
void k3o_set_threads(int n) { g_threads = n > 0 ? n : 1; }

/* ---------------------------------------------------------------------- */
/* Element formats                                                         */
/* ---------------------------------------------------------------------- */

/* The 16-entry E2M1 table: a weight is a 4-bit code indexing a 16-entry
 * table ([A176] "The four reductions"; [SAT] "Reduction one"). The pages do
 * not print the table; this is the OCP Microscaling E2M1 element format
 * (sign bit, two exponent bits with bias 1, one mantissa bit). Code 8 is -0.
 */
static const double E2M1[16] = {0.0,  0.5,  1.0,  1.5,  2.0,  3.0,  4.0,  6.0,
                                -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0};

double k3o_e2m1(int code) { return E2M1[code & 15]; }

/* E8M0 shared exponent: one 8-bit exponent per 32 weights ([A176] "The four
 * reductions"). Value 2^(e-127) (bias 127, the pages do not print it); byte
 * 255 is the format's NaN ([A176] "What byte-identical actually costs"). */
double k3o_e8m0(int e) {
  if (e == 255) return NAN;
  return ldexp(1.0, e - 127);
}

double k3o_bf16_to_f64(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t k3o_f32_to_bf16(float f) {
  /* Round to nearest, ties to even, on the 16 discarded bits. */
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x40u);
  const uint32_t hi = u >> 16, lo = u & 0xFFFFu;
  uint32_t r = hi;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) r = hi + 1u;
  return (uint16_t)r;
}

/* Element j of row r: low nibble for even j, high nibble for odd j
 * ([ZOR] "What are the four reductions, and why is the answer unchanged?":
 * the low nibble is the even element). */
static int code_at(const uint8_t *nib, int cols, int r, int j) {
  const uint8_t byte = nib[(size_t)r * (size_t)(cols / 2) + (size_t)(j / 2)];
  return (j % 2 == 0) ? (byte & 15) : (byte >> 4);
}

static int scale_at(const uint8_t *sc, int cols, int r, int j) {
  return sc[(size_t)r * (size_t)(cols / 32) + (size_t)(j / 32)];
}

/* ---------------------------------------------------------------------- */
/* MXFP4 GEMV                                                              */
/* ---------------------------------------------------------------------- */

/* y[r] = sum over groups g of 2^(e_g - 127) * (sum over the 32 elements i of
 * the group of E2M1(code_i) * x_i), read straight from the packed bytes:
 * each group is summed under its own double accumulator, its one scale is
 * applied after the group's dot product, and a group whose scale byte is 255
 * contributes nothing ([SAT] "Reduction one" (kernel comment and the
 * paragraph after it); [SAT] "A floating-point contract, not a convention",
 * MXFP4 exception; [A176] "What byte-identical actually costs").
 * Only group == 32 is described; anything else is refused. */
int k3o_mxfp4_gemv(const uint8_t *nib, const uint8_t *sc, int rows, int cols,
                   int group, const double *x, double *y) {
  if (!nib || !sc || !x || !y) return 1;
  if (group != 32 || cols <= 0 || cols % 32 != 0 || rows < 0) return 2;
  const int ngroups = cols / 32;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int r = 0; r < rows; r++) {
    double acc = 0.0;
    for (int g = 0; g < ngroups; g++) {
      const int e = scale_at(sc, cols, r, 32 * g);
      if (e == 255) continue; /* NaN scale: the group contributes nothing */
      double sub = 0.0;
      for (int i = 0; i < 32; i++) {
        const int j = 32 * g + i;
        sub += E2M1[code_at(nib, cols, r, j)] * x[j];
      }
      acc += sub * k3o_e8m0(e);
    }
    y[r] = acc;
  }
  return 0;
}

int k3o_mxfp4_dequant(const uint8_t *nib, const uint8_t *sc, int rows,
                      int cols, int group, double *W) {
  if (!nib || !sc || !W) return 1;
  if (group != 32 || cols <= 0 || cols % 32 != 0 || rows < 0) return 2;
  for (int r = 0; r < rows; r++)
    for (int j = 0; j < cols; j++) {
      const int e = scale_at(sc, cols, r, j);
      W[(size_t)r * cols + j] =
          (e == 255) ? 0.0 : E2M1[code_at(nib, cols, r, j)] * k3o_e8m0(e);
    }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Expert FFN                                                              */
/* ---------------------------------------------------------------------- */

/* SiLU(v) = v * sigmoid(v) = v / (1 + e^-v). The pages name their activation
 * but print no formula for it ([A176] "What byte-identical actually costs");
 * the expert FFN here is SwiGLU: h = SiLU(gate . x) * (up . x). */
double k3o_silu(double v) { return v / (1.0 + exp(-v)); }

/* One routed expert: three MXFP4 matrices, 3 * hidden * inter parameters
 * ([SAT] "Reduction one": one expert is 33,030,144 parameters = 3*7168*1536).
 * g = W_gate x, u = W_up x, h = SiLU(g) * u (kept in double), y = W_down h. */
int k3o_expert_swiglu(const k3o_expert *E, int hidden, int inter,
                      const double *x, double *h, double *y) {
  if (!E || !x || !y) return 1;
  double *g = (double *)malloc(sizeof(double) * (size_t)inter);
  double *u = (double *)malloc(sizeof(double) * (size_t)inter);
  double *hh = h ? h : (double *)malloc(sizeof(double) * (size_t)inter);
  int rc = (g && u && hh) ? 0 : 1;
  if (!rc) rc = k3o_mxfp4_gemv(E->gate_nib, E->gate_sc, inter, hidden, 32, x, g);
  if (!rc) rc = k3o_mxfp4_gemv(E->up_nib, E->up_sc, inter, hidden, 32, x, u);
  if (!rc) {
    for (int i = 0; i < inter; i++) hh[i] = k3o_silu(g[i]) * u[i];
    rc = k3o_mxfp4_gemv(E->down_nib, E->down_sc, hidden, inter, 32, hh, y);
  }
  free(g);
  free(u);
  if (!h) free(hh);
  return rc;
}

/* ---------------------------------------------------------------------- */
/* Router                                                                  */
/* ---------------------------------------------------------------------- */

/* Router logits l_e = sum_k x_k * R[e][k] over bf16 operands; routers stay
 * in the resident bf16 set ([ZOR] "How does a 2.78-trillion-parameter model
 * fit in 8 GB?"). Each product of two bf16 values is exact in double; the sum
 * runs sequentially over k in double. */
int k3o_router_logits(const uint16_t *x, const uint16_t *R, int n_experts,
                      int hidden, double *logits) {
  if (!x || !R || !logits) return 1;
  if (n_experts <= 0 || hidden <= 0) return 2;
  for (int e = 0; e < n_experts; e++) {
    double acc = 0.0;
    for (int k = 0; k < hidden; k++)
      acc += k3o_bf16_to_f64(x[k]) *
             k3o_bf16_to_f64(R[(size_t)e * (size_t)hidden + (size_t)k]);
    logits[e] = acc;
  }
  return 0;
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Selection and weights. The routing bias steers selection only: top-k is
 * taken on sigmoid(l) + bias, while the combine weights are the unbiased
 * sigmoid scores ([ZOR] "How is the C engine actually built?", invariant 3).
 * Without a bias the key is l itself (sigmoid is strictly increasing, so the
 * selected set is the same and no ties arise from saturation). Ties go to the
 * lower expert index; idx is in descending key order. Weights are
 * renormalised to sum to one: w_j = s_j / sum s (reading: the pages do not
 * state renormalisation; no further scale factor). */
int k3o_topk(const double *logits, const double *bias, int n, int k,
             int32_t *idx, double *w) {
  if (!logits || !idx || !w) return 1;
  if (n <= 0 || k < 1 || k > n) return 2;
  double *key = (double *)malloc(sizeof(double) * (size_t)n);
  char *taken = (char *)calloc((size_t)n, 1);
  if (!key || !taken) {
    free(key);
    free(taken);
    return 1;
  }
  for (int e = 0; e < n; e++)
    key[e] = bias ? sigmoid(logits[e]) + bias[e] : logits[e];
  for (int j = 0; j < k; j++) {
    int best = -1;
    for (int e = 0; e < n; e++) {
      if (taken[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e; /* strict: lower index wins ties */
    }
    taken[best] = 1;
    idx[j] = best;
  }
  double sum = 0.0;
  for (int j = 0; j < k; j++) {
    w[j] = sigmoid(logits[idx[j]]);
    sum += w[j];
  }
  for (int j = 0; j < k; j++) w[j] = w[j] / sum;
  free(key);
  free(taken);
  return 0;
}

/* y = sum_j w_j * ye[j], summed in rank order j = 0..k-1. */
int k3o_combine(const double *w, const double *ye, int k, int hidden,
                double *y) {
  if (!w || !ye || !y) return 1;
  for (int i = 0; i < hidden; i++) {
    double acc = 0.0;
    for (int j = 0; j < k; j++) acc += w[j] * ye[(size_t)j * hidden + i];
    y[i] = acc;
  }
  return 0;
}

static int expert_ok(const k3o_expert *E) {
  return E->gate_nib && E->gate_sc && E->up_nib && E->up_sc && E->down_nib &&
         E->down_sc;
}

/* Routed experts of one token, from its logits row. */
static int route_and_mix(const uint16_t *x, const double *logits,
                         const double *bias, const k3o_expert *experts,
                         int n_experts, int hidden, int inter, int k,
                         double *y, int32_t *idx, double *w) {
  int rc = k3o_topk(logits, bias, n_experts, k, idx, w);
  if (rc) return rc;
  double *xd = (double *)malloc(sizeof(double) * (size_t)hidden);
  double *ye = (double *)malloc(sizeof(double) * (size_t)hidden * (size_t)k);
  if (!xd || !ye) rc = 1;
  for (int i = 0; !rc && i < hidden; i++) xd[i] = k3o_bf16_to_f64(x[i]);
  for (int j = 0; !rc && j < k; j++) {
    const k3o_expert *E = &experts[idx[j]];
    if (!expert_ok(E)) {
      rc = 1;
      break;
    }
    rc = k3o_expert_swiglu(E, hidden, inter, xd, NULL, ye + (size_t)j * hidden);
  }
  if (!rc) rc = k3o_combine(w, ye, k, hidden, y);
  free(xd);
  free(ye);
  return rc;
}

/* One decode token: router GEMV, sigmoid top-k, the selected experts, the
 * weighted sum ([ZOR] "How is the C engine actually built?"; 16 of 896
 * experts fire per token, [A176] opening section). */
int k3o_moe_layer(const uint16_t *x, const uint16_t *R,
                  const k3o_expert *experts, int n_experts, int hidden,
                  int inter, int k, double *y, int32_t *idx, double *w) {
  if (!x || !R || !experts || !y || !idx || !w) return 1;
  if (hidden % 32 || inter % 32 || k < 1 || k > n_experts) return 2;
  double *logits = (double *)malloc(sizeof(double) * (size_t)n_experts);
  if (!logits) return 1;
  int rc = k3o_router_logits(x, R, n_experts, hidden, logits);
  if (!rc)
    rc = route_and_mix(x, logits, NULL, experts, n_experts, hidden, inter, k,
                       y, idx, w);
  free(logits);
  return rc;
}

int k3o_moe_from_logits(const uint16_t *X, const double *logits,
                        const double *bias, const k3o_expert *experts, int T,
                        int n_experts, int hidden, int inter, int k,
                        double *Y, int32_t *idx, double *w) {
  if (!X || !logits || !experts || !Y || !idx || !w) return 1;
  if (hidden % 32 || inter % 32 || k < 1 || k > n_experts || T < 0) return 2;
  for (int t = 0; t < T; t++) {
    const int rc = route_and_mix(X + (size_t)t * hidden,
                                 logits + (size_t)t * n_experts, bias, experts,
                                 n_experts, hidden, inter, k,
                                 Y + (size_t)t * hidden, idx + (size_t)t * k,
                                 w + (size_t)t * k);
    if (rc) return rc;
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Shared experts                                                          */
/* ---------------------------------------------------------------------- */

/* One shared expert: a SwiGLU FFN whose three matrices are bf16 and stay in
 * the resident set, run on every token beside the routed ones ([ZOR] "How
 * does a 2.78-trillion-parameter model fit in 8 GB?": two shared experts per
 * layer, classed with the always-on bf16 weights). The pages give neither
 * their width nor how their output joins the routed one; the reading taken
 * here: the routed expert's shapes, and y = routed mix + the shared outputs,
 * unweighted. g = W_gate x, u = W_up x, h = SiLU(g) * u, y = W_down h, all in
 * double over the exactly widened bf16 weights; sums run in index order. */
static double dot_bf16_row(const uint16_t *row, const double *v, int n) {
  double acc = 0.0;
  for (int c = 0; c < n; c++) acc += k3o_bf16_to_f64(row[c]) * v[c];
  return acc;
}

int k3o_shared_expert(const k3o_shared *S, int hidden, int inter,
                      const double *x, double *h, double *y) {
  if (!S || !S->gate || !S->up || !S->down || !x || !y) return 1;
  if (hidden <= 0 || inter <= 0) return 2;
  double *hh = h ? h : (double *)malloc(sizeof(double) * (size_t)inter);
  if (!hh) return 1;
  for (int i = 0; i < inter; i++) {
    const double g = dot_bf16_row(S->gate + (size_t)i * hidden, x, hidden);
    const double u = dot_bf16_row(S->up + (size_t)i * hidden, x, hidden);
    hh[i] = k3o_silu(g) * u;
  }
  for (int r = 0; r < hidden; r++)
    y[r] = dot_bf16_row(S->down + (size_t)r * inter, hh, inter);
  if (!h) free(hh);
  return 0;
}

/* The decode layer with shared experts: the routed layer's y, then the
 * shared experts' outputs added in order s = 0, 1, ... */
int k3o_moe_layer_shared(const uint16_t *x, const uint16_t *R,
                         const k3o_expert *experts, int n_experts, int hidden,
                         int inter, int k, const k3o_shared *shared,
                         int n_shared, int inter_shared, double *y,
                         int32_t *idx, double *w) {
  if (!shared && n_shared > 0) return 1;
  if (n_shared < 0) return 2;
  int rc = k3o_moe_layer(x, R, experts, n_experts, hidden, inter, k, y, idx, w);
  if (rc) return rc;
  double *xd = (double *)malloc(sizeof(double) * (size_t)hidden);
  double *ys = (double *)malloc(sizeof(double) * (size_t)hidden);
  if (!xd || !ys) rc = 1;
  for (int i = 0; !rc && i < hidden; i++) xd[i] = k3o_bf16_to_f64(x[i]);
  for (int s = 0; !rc && s < n_shared; s++) {
    rc = k3o_shared_expert(&shared[s], hidden, inter_shared, xd, NULL, ys);
    for (int r = 0; !rc && r < hidden; r++) y[r] += ys[r];
  }
  free(xd);
  free(ys);
  return rc;
}

/* Pairs (t, j) grouped by expert, ascending token inside each expert. */
int k3o_permute(const int32_t *idx, int T, int k, int n_experts,
                int32_t *counts, int32_t *offsets, int32_t *pair_token,
                int32_t *pair_slot) {
  if (!idx || !counts || !offsets || !pair_token || !pair_slot) return 1;
  int pos = 0;
  for (int e = 0; e < n_experts; e++) {
    offsets[e] = pos;
    counts[e] = 0;
    for (int t = 0; t < T; t++)
      for (int j = 0; j < k; j++)
        if (idx[(size_t)t * k + j] == e) {
          pair_token[pos] = t;
          pair_slot[pos] = j;
          pos++;
          counts[e]++;
        }
  }
  return pos == T * k ? 0 : 2;
}

/* ---------------------------------------------------------------------- */
/* MXFP4 activation quantiser and MXFP4 x MXFP4 product (prefill)          */
/* ---------------------------------------------------------------------- */

/* Round a scaled value to the nearest E2M1 code, ties to the even code
 * (mantissa bit 0), saturating at +-6; a result of magnitude 0 is written as
 * code 0. The pages describe no quantiser ([A176] "What is missing or worth
 * watching" says the engine has none): the rule here is the OCP MX
 * conversion (largest power of two not above max|v|, minus the E2M1 maximum
 * exponent 2), and its choice is parity unpinned. */
static int e2m1_round(double t) {
  const double mag = fabs(t);
  int best = 0;
  for (int m = 1; m < 8; m++) {
    const double d = fabs(mag - E2M1[m]), db = fabs(mag - E2M1[best]);
    if (d < db || (d == db && (m % 2 == 0))) best = m;
  }
  if (best == 0) return 0;
  return (t < 0) ? (8 | best) : best;
}

int k3o_mxfp4_quant(const double *v, int rows, int cols, uint8_t *nib,
                    uint8_t *sc) {
  if (!v || !nib || !sc) return 1;
  if (cols <= 0 || cols % 32 != 0 || rows < 0) return 2;
  for (int r = 0; r < rows; r++)
    for (int g = 0; g < cols / 32; g++) {
      const double *blk = v + (size_t)r * cols + (size_t)g * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; i++)
        if (fabs(blk[i]) > amax) amax = fabs(blk[i]);
      int codes[32] = {0};
      int e = 0;
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1) */
        int E = (ex - 1) - 2;
        if (E < -127) E = -127;
        if (E > 127) E = 127;
        e = E + 127;
        for (int i = 0; i < 32; i++) codes[i] = e2m1_round(ldexp(blk[i], -E));
      }
      sc[(size_t)r * (cols / 32) + g] = (uint8_t)e;
      for (int i = 0; i < 32; i += 2)
        nib[(size_t)r * (cols / 2) + (size_t)g * 16 + i / 2] =
            (uint8_t)(codes[i] | (codes[i + 1] << 4));
    }
  return 0;
}

/* C[m][n] = sum over groups of 2^(ea-127) 2^(ew-127) * sum_i a_i w_i, both
 * operands MXFP4 along K, skipping a group where either scale is 255. */
int k3o_mxfp4_matmul(const uint8_t *a_nib, const uint8_t *a_sc, int M,
                     const uint8_t *w_nib, const uint8_t *w_sc, int N, int K,
                     double *C) {
  if (!a_nib || !a_sc || !w_nib || !w_sc || !C) return 1;
  if (K <= 0 || K % 32 != 0 || M < 0 || N < 0) return 2;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int m = 0; m < M; m++)
    for (int n = 0; n < N; n++) {
      double acc = 0.0;
      for (int g = 0; g < K / 32; g++) {
        const int ea = scale_at(a_sc, K, m, 32 * g);
        const int ew = scale_at(w_sc, K, n, 32 * g);
        if (ea == 255 || ew == 255) continue;
        double sub = 0.0;
        for (int i = 0; i < 32; i++) {
          const int j = 32 * g + i;
          sub += E2M1[code_at(a_nib, K, m, j)] * E2M1[code_at(w_nib, K, n, j)];
        }
        acc += sub * k3o_e8m0(ea) * k3o_e8m0(ew);
      }
      C[(size_t)m * N + n] = acc;
    }
  return 0;
}
