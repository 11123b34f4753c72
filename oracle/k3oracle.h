/*
 * k3oracle — plain, slow, fp64 CPU reference of the MXFP4 routed-expert path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this code; it exists so tests, the smoke check and the CPU-baseline leg
 * of the benchmark can check the GPU library against an independent
 * definition. It shares no code, header, table or helper with the GPU library.
 *
 * Sources (web pages describing the kimi-k3-in-c engine):
 *  [A176] "kimi-k3-in-c: A 176 KB Engine That Runs a 2.78T-Parameter MoE in
 *         8 GB of RAM" (aniketkarneai.com)
 *  [SAT]  "kimi-k3-in-c" explainer (ai.thesatyajit.com/articles/kimi-k3-in-c)
 *  [ZOR]  "Running Kimi K3 locally: activation sparsity as architecture"
 *         (zorost.com)
 * Where the pages are silent the reading taken is named in each function's
 * comment and listed in the design doc's readings table.
 *
 * Canonical MXFP4 layout (the layout of the checkpoint bytes as the pages
 * describe them): a matrix W[rows][cols] is
 *   nib[rows][cols/2]  byte b of a row holds element 2b in its LOW nibble and
 *                      element 2b+1 in its HIGH nibble  ([ZOR] "What are the
 *                      four reductions..."; [A176] "What byte-identical
 *                      actually costs")
 *   sc[rows][cols/32]  one E8M0 exponent byte per 32 consecutive elements of
 *                      a row ([SAT] "Reduction one").
 *
 * Return codes: 0 ok, 1 bad argument (NULL pointer), 2 unsupported
 * configuration (group != 32, cols % 32 != 0, k out of range, ...).
 *
 * Parity status: every function below is pinned by tests under tests/ against
 * facts independent of this file, except k3o_mxfp4_quant's choice of scale
 * and rounding rule, which the pages do not describe ("parity unpinned" for
 * the rule itself; its invariants are pinned).
 */
#ifndef K3ORACLE_H
#define K3ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- element formats -------------------------------------------------- */
double k3o_e2m1(int code);           /* 4-bit E2M1 code -> value            */
double k3o_e8m0(int e);              /* 2^(e-127); NaN for e == 255         */
double k3o_bf16_to_f64(uint16_t b);  /* exact widening                      */
uint16_t k3o_f32_to_bf16(float f);   /* round to nearest even               */

/* ---- MXFP4 matrix-vector product (packed, never dequantised) --------- */
int k3o_mxfp4_gemv(const uint8_t *nib, const uint8_t *sc, int rows, int cols,
                   int group, const double *x, double *y);
/* Alternative path used only by checks: expand W to doubles. */
int k3o_mxfp4_dequant(const uint8_t *nib, const uint8_t *sc, int rows,
                      int cols, int group, double *W);

/* ---- routed expert (SwiGLU FFN) -------------------------------------- */
typedef struct {
  const uint8_t *gate_nib, *gate_sc; /* [inter][hidden] */
  const uint8_t *up_nib, *up_sc;     /* [inter][hidden] */
  const uint8_t *down_nib, *down_sc; /* [hidden][inter] */
} k3o_expert;

double k3o_silu(double v);
int k3o_expert_swiglu(const k3o_expert *E, int hidden, int inter,
                      const double *x, double *h /* [inter] or NULL */,
                      double *y /* [hidden] */);

/* ---- router ------------------------------------------------------------ */
int k3o_router_logits(const uint16_t *x, const uint16_t *R, int n_experts,
                      int hidden, double *logits);
int k3o_topk(const double *logits, const double *bias /* or NULL */, int n,
             int k, int32_t *idx, double *w);
int k3o_combine(const double *w, const double *ye /* [k][hidden] */, int k,
                int hidden, double *y);

/* ---- whole layer ------------------------------------------------------- */
/* One token: router GEMV -> top-k -> experts -> combine. experts[e] must be
 * filled for every selected e (others may hold NULL pointers). */
int k3o_moe_layer(const uint16_t *x, const uint16_t *R,
                  const k3o_expert *experts, int n_experts, int hidden,
                  int inter, int k, double *y, int32_t *idx, double *w);
/* T tokens routed from given logits [T][n_experts]. */
int k3o_moe_from_logits(const uint16_t *X, const double *logits,
                        const double *bias, const k3o_expert *experts, int T,
                        int n_experts, int hidden, int inter, int k,
                        double *Y, int32_t *idx, double *w);
/* Token->expert permutation: pairs (t, j) stably sorted by (expert, token). */
int k3o_permute(const int32_t *idx, int T, int k, int n_experts,
                int32_t *counts, int32_t *offsets, int32_t *pair_token,
                int32_t *pair_slot);

/* ---- shared experts (bf16, every token) -------------------------------- */
typedef struct {
  const uint16_t *gate, *up; /* bf16 [inter][hidden], row-major */
  const uint16_t *down;      /* bf16 [hidden][inter], row-major */
} k3o_shared;
int k3o_shared_expert(const k3o_shared *S, int hidden, int inter,
                      const double *x, double *h /* [inter] or NULL */,
                      double *y /* [hidden] */);
/* The routed layer (k3o_moe_layer) plus the n_shared shared experts'
 * outputs, added in order. */
int k3o_moe_layer_shared(const uint16_t *x, const uint16_t *R,
                         const k3o_expert *experts, int n_experts, int hidden,
                         int inter, int k, const k3o_shared *shared,
                         int n_shared, int inter_shared, double *y,
                         int32_t *idx, double *w);

/* ---- MXFP4 activation quantiser (prefill) ------------------------------ */
int k3o_mxfp4_quant(const double *v, int rows, int cols, uint8_t *nib,
                    uint8_t *sc);
/* C[m][n] = A[m] . W[n] with both operands canonical MXFP4 along K (A: M
 * activation rows, W: N weight rows), group-then-scale in double. */
int k3o_mxfp4_matmul(const uint8_t *a_nib, const uint8_t *a_sc, int M,
                     const uint8_t *w_nib, const uint8_t *w_sc, int N, int K,
                     double *C /* [M][N] */);

/* Threads used by the row loops (results do not depend on it). */
void k3o_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
