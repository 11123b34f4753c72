/*
 * k3moe — MXFP4 routed-expert MoE path for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libk3moe.so. Every pointer named *_d, and every tensor argument of
 * a compute call, is a DEVICE pointer; *_host functions take host pointers.
 * bf16 values travel as uint16_t bit patterns. Nothing here allocates: the
 * caller owns every buffer, including the workspace. Compute calls validate
 * all arguments on the host before anything is enqueued (on error nothing is
 * launched), then enqueue asynchronously on `stream` and never synchronise.
 * Calls on different streams with different outputs and workspaces may be
 * issued concurrently, from any host threads. The decode layer's expert
 * launch (k3_moe_layer, _ex, _noalloc, _shared, _cached, and
 * k3_moe_layer_from_logits with T = 1 and no bias) and k3_expert_swiglu_ws
 * need their whole grid resident at once, so the library orders those
 * launches on one device. While they all go to one
 * stream, the stream orders them. The first one issued on a second stream
 * blocks the calling thread until the device is idle; from then on an event
 * is recorded after each of them, and one issued on another stream than
 * the previous one waits for it on the device. Every other launch may
 * overlap with anything.
 *
 * Sources (web pages describing the kimi-k3-in-c engine), cited below as:
 *  [A176] "kimi-k3-in-c: A 176 KB Engine That Runs a 2.78T-Parameter MoE in
 *         8 GB of RAM"
 *  [SAT]  ai.thesatyajit.com, "kimi-k3-in-c" explainer
 *  [ZOR]  "Running Kimi K3 locally: activation sparsity as architecture"
 *
 * MXFP4: a weight is a 4-bit E2M1 code; 32 consecutive weights of a row share
 * one 8-bit E8M0 exponent e meaning 2^(e-127); 0.53125 bytes per weight
 * ([A176] "The four reductions"). Exponent byte 255 (the format's NaN) makes
 * its group contribute nothing, even where the activations are not finite
 * ([A176] "What byte-identical actually costs"). Exact-domain contract: for
 * exponent bytes in [2, 252] every decoded weight is an fp32 normal number;
 * outside that range results follow fp32 (under/overflow) and are not gated.
 *
 * Canonical layout (the checkpoint's bytes): nib[rows][cols/2] with element
 * 2b in the LOW nibble of byte b and element 2b+1 in the high nibble ([ZOR]
 * "What are the four reductions, and why is the answer unchanged?"), and
 * sc[rows][cols/32]. The compute calls read the device tile layout written by
 * k3_mxfp4_pack / k3_expert_pack (a one-time re-tiling, see k3_mxfp4_pack).
 *
 * Status codes: K3_ERR_ARG for a NULL or misaligned pointer (all device
 * pointers must be 16-byte aligned); K3_ERR_CONFIG for dimensions the path
 * does not support or that contradict each other (the call names them in
 * k3_last_error; nothing is defaulted, following the pages' config reader
 * that refuses to guess, [A176] "What byte-identical actually costs");
 * K3_ERR_MEMORY when the workspace is smaller than the call needs (the
 * message gives both sizes, so the caller sees that more memory, not a
 * different configuration, would serve the call; the pages report memory
 * budgets the same way, [A176] "The interesting design decisions");
 * K3_ERR_DEVICE when the HIP runtime
 * reports a launch or runtime error.
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t; NULL means the default stream. */
typedef struct ihipStream_t *k3_stream_t;

typedef int k3_status;
#define K3_OK 0
#define K3_ERR_ARG 1
#define K3_ERR_CONFIG 2
#define K3_ERR_MEMORY 3
#define K3_ERR_DEVICE 4

/* Largest expert count and top-k the routing kernels handle, and the largest
 * expert dimensions (the expert kernels keep one activation vector in LDS). */
#define K3_MAX_EXPERTS 4096
#define K3_MAX_TOPK 64
#define K3_MAX_SHARED 8
#define K3_MAX_HIDDEN 16384
#define K3_MAX_INTER 4096

const char *k3_strerror(k3_status s);
/* Detail of the last failed call on the calling thread ("" if none). */
const char *k3_last_error(void);
int k3_abi_version(void);

/* ------------------------------------------------------------------------
 * Layout. A matrix W[rows][cols] (cols % 32 == 0) is stored as ceil(rows/64)
 * tiles of 64 rows. With G = cols/32 groups and G4 = ceil(G/4), tile t is G4
 * quad blocks of 4352 bytes; quad block q of tile t holds, for l = 0..63:
 *   bytes [1024*b + 16*l, +16)  the 16 canonical bytes (32 codes) of group
 *                               g = 4q+b of row 64t + l (zero for g >= G);
 *   byte  4096 + 4*l + b        the exponent byte of that group (0 for
 *                               g >= G).
 * so lane l of a wave reads its row's group g with one 16-byte load, the
 * wave's 64 loads are one contiguous KiB, and a wave walking a row range
 * reads one contiguous stream. Rows past `rows` are zero codes with exponent
 * byte 0. Tile size 4352*G4 bytes (no padding when G % 4 == 0). Groups of 32
 * are 16 packed bytes ([SAT] "Reduction one"), which is what makes a group
 * one 128-bit load.
 * ---------------------------------------------------------------------- */
size_t k3_mxfp4_packed_bytes(int rows, int cols);
/* Host re-tiling; tiles must hold k3_mxfp4_packed_bytes(rows, cols). */
k3_status k3_mxfp4_pack_host(const uint8_t *nib, const uint8_t *sc, int rows,
                             int cols, uint8_t *tiles);
k3_status k3_mxfp4_unpack_host(const uint8_t *tiles, int rows, int cols,
                               uint8_t *nib, uint8_t *sc);
/* Same re-tiling on the device (all pointers device). */
k3_status k3_mxfp4_pack(const uint8_t *nib_d, const uint8_t *sc_d, int rows,
                        int cols, uint8_t *tiles_d, k3_stream_t stream);
k3_status k3_mxfp4_unpack(const uint8_t *tiles_d, int rows, int cols,
                          uint8_t *nib_d, uint8_t *sc_d, k3_stream_t stream);

/* A routed expert ([SAT] "Reduction one": three MXFP4 matrices, gate and up
 * [inter][hidden], down [hidden][inter]) is one blob:
 *   [gate/up tiles][down tiles]
 * The gate/up part is the tile layout above over 2*inter virtual rows in
 * which tile t holds gate rows 32t..32t+31 in lanes 0..31 and up rows
 * 32t..32t+31 in lanes 32..63 (so one tile yields both inputs of the SwiGLU
 * for 32 rows). The down part is the plain tile layout of W_down.
 * hidden % 32 == 0 and inter % 32 == 0 are required, hidden <= K3_MAX_HIDDEN,
 * inter <= K3_MAX_INTER. */
size_t k3_expert_packed_bytes(int hidden, int inter);
k3_status k3_expert_pack_host(const uint8_t *gate_nib, const uint8_t *gate_sc,
                              const uint8_t *up_nib, const uint8_t *up_sc,
                              const uint8_t *down_nib, const uint8_t *down_sc,
                              int hidden, int inter, uint8_t *expert);
k3_status k3_expert_pack(const uint8_t *gate_nib_d, const uint8_t *gate_sc_d,
                         const uint8_t *up_nib_d, const uint8_t *up_sc_d,
                         const uint8_t *down_nib_d, const uint8_t *down_sc_d,
                         int hidden, int inter, uint8_t *expert_d,
                         k3_stream_t stream);

/* ------------------------------------------------------------------------
 * y[rows] = W[rows][cols] . x[cols] read straight from the packed bytes,
 * never expanded to floats in memory ([SAT] "Reduction one"). The codes go
 * to gfx950's block-scaled matrix instruction as they are stored (E2M1, each
 * group's exponent byte as its block scale), against x cut into six 4-bit
 * fixed-point digits per value below the largest exponent of its group of
 * 32: a bf16 value within 2^-16 of its group's largest is carried exactly,
 * any other value to within half an fp32 ulp of the group's largest. Every
 * block sum is exact and the sums accumulate in fp32; exponent 255
 * contributes nothing. A workgroup whose x groups hold a non-finite value
 * or a largest value outside [2^-87, 2^122) multiplies on the vector ALU
 * instead: the group's codes converted in registers, multiplied by x in
 * fp32, the exponent applied once to the group's sum. fp32 accumulation in
 * a fixed order: each row is reduced by one workgroup along a fixed tree,
 * so results are bit-identical from run to run on one device (the pages'
 * fixed-order rule, [SAT] "A floating-point contract, not a convention").
 * x fp32 [cols], tiles from k3_mxfp4_pack, y fp32 [rows]. No workspace.
 * ---------------------------------------------------------------------- */
k3_status k3_mxfp4_gemv(const float *x, const uint8_t *tiles, int rows,
                        int cols, float *y, k3_stream_t stream);

/* One routed expert, SwiGLU: g = W_gate x, u = W_up x, h = SiLU(g) * u
 * (fp32, not rounded to bf16), y = W_down h. x bf16 [hidden]; expert from
 * k3_expert_pack; y fp32 [hidden]; h fp32 [inter] receives h. Same product
 * as k3_mxfp4_gemv. */
k3_status k3_expert_swiglu(const uint16_t *x, const uint8_t *expert,
                           int hidden, int inter, float *y, float *h,
                           k3_stream_t stream);

/* The same expert in one launch over every compute unit, for a lone expert
 * (the two launches above occupy only as many compute units as the matrix
 * has 64-row tiles). The gate/up tiles are cut along K into chunks, one per
 * workgroup; their row partials go to the workspace, and the workgroups that
 * own down tiles (whose first bytes they load before the gate/up work) sum
 * each row's partials in chunk order, form h and multiply their tile by it.
 * The products are the vector-ALU form described at k3_mxfp4_gemv (one
 * expert is bound by its chain of memory round trips, not by arithmetic),
 * and the summation order differs from k3_expert_swiglu's, so the two differ
 * in the last bits; each is bit-identical from run to run on one device. h fp32
 * [inter] is optional (NULL: not written). ws: at least
 * k3_expert_swiglu_workspace_bytes(hidden, inter) bytes; calls sharing a
 * workspace must not overlap. The launch needs its whole grid resident; it
 * is ordered with the decode layer's expert launch across streams (top of
 * this file). While the stream is being captured it runs the two launches
 * of k3_expert_swiglu instead (same bits as those). */
size_t k3_expert_swiglu_workspace_bytes(int hidden, int inter);
k3_status k3_expert_swiglu_ws(const uint16_t *x, const uint8_t *expert,
                              int hidden, int inter, float *y, float *h,
                              void *ws, size_t ws_bytes, k3_stream_t stream);

/* The two stages of k3_expert_swiglu over k routing slots of one token, and
 * the weighted combine, as separate calls (k3_moe_layer runs exactly these):
 *   k3_expert_gate_up:  h[j][inter] = SiLU(W_gate(e_j) x) * (W_up(e_j) x)
 *   k3_expert_down:     yp[j][hidden] = W_down(e_j) h[j]
 *   k3_moe_combine:     y[i] = sum_{j<k} w[j] * yp[j][i] in rank order (fp32),
 *                       y_f32 (optional) the fp32 value, y bf16 (RNE).
 * with e_j = idx[j] (device int32 [k], each in [0, n_experts)) and experts the
 * device pointer table of k3_moe_layer. 1 <= k <= K3_MAX_TOPK. */
k3_status k3_expert_gate_up(const uint16_t *x, const uint8_t *const *experts,
                            const int32_t *idx, int k, int hidden, int inter,
                            float *h, k3_stream_t stream);
/* The first stage as k3_moe_layer runs it: top-k of one token's logits
 * (device fp64 [n_experts], no bias, n_experts <= 1024; as k3_router_topk)
 * inside the gate/up launch, writing idx int32 [k] and w fp32 [k] and
 * h[j][inter] as k3_expert_gate_up. */
k3_status k3_expert_gate_up_routed(const uint16_t *x, const double *logits,
                                   const uint8_t *const *experts, int n_experts,
                                   int k, int hidden, int inter, float *h,
                                   int32_t *idx, float *w, k3_stream_t stream);
k3_status k3_expert_down(const float *h, const uint8_t *const *experts,
                         const int32_t *idx, int k, int hidden, int inter,
                         float *yp, k3_stream_t stream);
k3_status k3_moe_combine(const float *yp, const float *w, int k, int hidden,
                         uint16_t *y, float *y_f32, k3_stream_t stream);

/* ------------------------------------------------------------------------
 * Router. logits[t][e] = sum_k x[t][k] * R[e][k] over bf16 operands, with
 * products and sums in fp64 (routers stay in the resident bf16 set, [ZOR]
 * "How does a 2.78-trillion-parameter model fit in 8 GB?"). x [T][hidden],
 * router_w [n_experts][hidden] row-major, logits fp64 [T][n_experts].
 * ---------------------------------------------------------------------- */
k3_status k3_router(const uint16_t *x, const uint16_t *router_w, int T,
                    int hidden, int n_experts, double *logits,
                    k3_stream_t stream);

/* Top-k per token. Key = logit without bias, sigmoid(logit) + bias[e] with
 * one; selection by key, ties to the lower expert index, idx in descending
 * key order. Weights from the UNBIASED scores s = sigmoid(logit),
 * renormalised w_j = s_j / sum s (the bias steers selection only, [ZOR]
 * "How is the C engine actually built?", invariant 3). Keys, sigmoid and the
 * sums are fp64. logits [T][n_experts] (fp64 or fp32 variant), bias fp32
 * [n_experts] or NULL, idx int32 [T][k], w fp32 [T][k].
 * 1 <= k <= min(n_experts, K3_MAX_TOPK), n_experts <= K3_MAX_EXPERTS. */
k3_status k3_router_topk(const double *logits, const float *bias, int T,
                         int n_experts, int k, int32_t *idx, float *w,
                         k3_stream_t stream);
k3_status k3_router_topk_f32(const float *logits, const float *bias, int T,
                             int n_experts, int k, int32_t *idx, float *w,
                             k3_stream_t stream);
/* k3_router_topk with the renormalised weights multiplied by routed_scale:
 * w_j = fp32((s_j / sum s) * routed_scale), the product in fp64. The pages
 * name the routing bias but no scale on the routed weights ([ZOR] "How is
 * the C engine actually built?", invariant 3), so the layer calls use 1; a
 * model with a routed scaling factor takes these weights into the
 * stage-by-stage calls (k3_expert_gate_up, k3_expert_down, k3_moe_combine).
 * routed_scale must be positive and finite (K3_ERR_CONFIG otherwise). */
k3_status k3_router_topk_scaled(const double *logits, const float *bias, int T,
                                int n_experts, int k, double routed_scale,
                                int32_t *idx, float *w, k3_stream_t stream);

/* ------------------------------------------------------------------------
 * Whole decode MoE layer for one token: router GEMV -> sigmoid top-k ->
 * the k selected SwiGLU experts -> y = sum_j w_j * y_j in rank order (fp32)
 * -> bf16 (round to nearest even). 16 of 896 experts per token in the
 * pages' model ([A176] opening section).
 *   x         bf16 [hidden]
 *   router_w  bf16 [n_experts][hidden]
 *   experts   device array of n_experts device pointers, experts[e] -> blob
 *             of k3_expert_pack for expert e
 *   y         bf16 [hidden]
 *   ws        workspace of >= k3_moe_workspace_bytes(1, n_experts, hidden,
 *             inter, k) bytes
 * k3_moe_layer_ex also writes (any may be NULL) y_f32 [hidden] (the value
 * before the bf16 cast), idx int32 [k], w fp32 [k], logits fp64 [n_experts].
 *
 * Two launches: the router, then the expert work (top-k, gate/up + SwiGLU,
 * down, combine) in one grid of one workgroup per compute unit whose stages
 * hand over through the workspace, marked with a per-call value (so the
 * workspace needs no initialisation, but calls that share one workspace
 * must not overlap). Its bits equal those of the stage-by-stage calls below
 * (k3_expert_gate_up_routed, k3_expert_down, k3_moe_combine), which are
 * what the layer runs while the stream is being captured into a graph or
 * for n_experts > 1024. Two such expert launches never overlap (see the top
 * of this file). Its internal waits are bounded: if the device cannot run
 * its whole grid at once for about a second (a kernel of another library,
 * on another stream, holding compute units all that time), it writes NaN
 * to y_f32 and 0x7FC0 (bf16 NaN) to y instead of hanging.
 * ---------------------------------------------------------------------- */
size_t k3_moe_workspace_bytes(int T, int n_experts, int hidden, int inter,
                              int k);
k3_status k3_moe_layer(const uint16_t *x, const uint16_t *router_w,
                       const uint8_t *const *experts, int n_experts,
                       int hidden, int inter, int k, uint16_t *y, void *ws,
                       size_t ws_bytes, k3_stream_t stream);
k3_status k3_moe_layer_ex(const uint16_t *x, const uint16_t *router_w,
                          const uint8_t *const *experts, int n_experts,
                          int hidden, int inter, int k, uint16_t *y,
                          float *y_f32, int32_t *idx, float *w,
                          double *logits, void *ws, size_t ws_bytes,
                          k3_stream_t stream);

/* ----------------------------------------------------------------------
 * k3_moe_layer_noalloc: k3_moe_layer_ex without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture,
 * serving loops, harnesses that forbid allocation). Same arguments, outputs,
 * kernels and bits as k3_moe_layer_ex. Its scratch is a static device array
 * of K3_NOALLOC_SCRATCH_BYTES inside the library, one per device, held until
 * the process ends; the call allocates nothing. Shapes whose scratch
 * (k3_moe_workspace_bytes(1, n_experts, hidden, inter, k)) exceeds it are
 * refused with K3_ERR_MEMORY (the 896-expert, 7168/1536, top-16 layer needs
 * about 0.58 MB). Every call on one device shares that device's array:
 * calls that overlap on one device (on different streams, or a call on
 * another stream before an earlier one finished) race on it and must be
 * ordered by the caller. Nothing in it needs clearing between calls (its
 * arrival slots carry a per-call value).
 * ---------------------------------------------------------------------- */
#define K3_NOALLOC_SCRATCH_BYTES (2u << 20)
k3_status k3_moe_layer_noalloc(const uint16_t *x, const uint16_t *router_w,
                               const uint8_t *const *experts, int n_experts,
                               int hidden, int inter, int k, uint16_t *y,
                               float *y_f32, int32_t *idx, float *w,
                               double *logits, k3_stream_t stream);

/* ------------------------------------------------------------------------
 * Batched decode: T tokens, each routed to k of n_experts experts; every
 * selected expert's packed bytes are read once for all of its tokens.
 *
 * k3_moe_permute: the T*k routing pairs p = t*k + j (expert idx[p], device
 * int32 [T][k]) sorted by expert, stably in pair order (token, then slot):
 *   counts[e]   pairs of expert e                     (device int32 [n])
 *   offsets[e]  start of expert e's run               (device int32 [n])
 *   pair_token[q], pair_slot[q]  token and slot of the q-th sorted pair
 *               (device int32 [T*k]).
 * Entries of idx outside [0, n_experts) are not placed. ws: device scratch
 * of k3_moe_permute_workspace_bytes(T, k) bytes. 1 <= k <= K3_MAX_TOPK,
 * T*k <= 2^20.
 *
 * k3_moe_layer_from_logits: for each token t, top-k of logits[t] (device
 * fp64 [T][n_experts]; bias optional as in k3_router_topk), then
 *   Y[t] = sum_j w[t][j] * SwiGLU_{idx[t][j]}(X[t])  in rank order j,
 * X bf16 [T][hidden]; Y bf16 [T][hidden] (RNE) and/or Y_f32 fp32
 * [T][hidden]; idx int32 [T][k] and w fp32 [T][k] optional outputs.
 * k3_moe_layer_batched: the same with the logits from the router
 * (k3_router of X against router_w bf16 [n_experts][hidden], no bias).
 * Both take a workspace of k3_moe_batched_workspace_bytes(T, n_experts,
 * hidden, inter, k) bytes. Each Y[t] is summed in an order fixed by the
 * routing of the whole batch, so reruns are bit-identical. One token
 * (T == 1) without a bias takes the single-token layer's expert launch (as
 * k3_moe_layer after its router; same workspace rules).
 * ---------------------------------------------------------------------- */
size_t k3_moe_permute_workspace_bytes(int T, int k);
k3_status k3_moe_permute(const int32_t *idx, int T, int k, int n_experts,
                         int32_t *counts, int32_t *offsets, int32_t *pair_token,
                         int32_t *pair_slot, void *ws, size_t ws_bytes,
                         k3_stream_t stream);
size_t k3_moe_batched_workspace_bytes(int T, int n_experts, int hidden,
                                      int inter, int k);
k3_status k3_moe_layer_from_logits(const uint16_t *X, const double *logits,
                                   const float *bias,
                                   const uint8_t *const *experts,
                                   int n_experts, int hidden, int inter, int k,
                                   int T, uint16_t *Y, float *Y_f32,
                                   int32_t *idx, float *w, void *ws,
                                   size_t ws_bytes, k3_stream_t stream);
k3_status k3_moe_layer_batched(const uint16_t *X, const uint16_t *router_w,
                               const uint8_t *const *experts, int n_experts,
                               int hidden, int inter, int k, int T, uint16_t *Y,
                               float *Y_f32, int32_t *idx, float *w, void *ws,
                               size_t ws_bytes, k3_stream_t stream);

/* ------------------------------------------------------------------------
 * Prefill: many tokens per expert, so the expert products are dense
 * contractions on gfx950's block-scaled FP4 matrix instruction with both
 * operands MXFP4. The pages' engine has no activation quantiser ([A176]
 * "What is missing or worth watching"); the rule used here: for each block
 * of 32 values along K, E = floor(log2 max|v|) - 2 clamped to [-127, 127],
 * exponent byte E + 127, codes = E2M1 nearest to v / 2^E with ties to the
 * even code (0, 1, 2, 4), saturating at 6; a code of magnitude 0 is code 0;
 * an all-zero block has exponent byte 0.
 *
 * k3_mxfp4_quantize_{f32,bf16}: v[rows][cols] (device) -> nib[rows][cols/2]
 * (element 2b in the low nibble of byte b) and sc[rows][cols/32].
 *
 * k3_moe_prefill: for T tokens X bf16 [T][hidden] routed by top-k of logits
 * (fp64 [T][n_experts], optional bias as in k3_router_topk): x is quantised,
 * every selected expert's gate/up stack is multiplied by its tokens' x, h =
 * SiLU(gate) * up (fp32) is quantised per 32 along inter, multiplied by the
 * down matrix, and Y[t] = sum_j w[t][j] * y_{idx[t][j]}(t) in rank order.
 * Y bf16 / Y_f32 fp32 [T][hidden]; idx int32 [T][k], w fp32 [T][k] optional.
 * Optional exports of h, indexed by sorted pair q (the order of
 * k3_moe_permute over idx): h_f32 fp32 [T*k][inter] before quantisation,
 * h_nib [T*k][inter/2] and h_sc [T*k][inter/32] (given together) after.
 * Workspace: k3_moe_prefill_workspace_bytes(T, n_experts, hidden, inter, k)
 * bytes, which include the fp32 partials [T*k][hidden].
 * ---------------------------------------------------------------------- */
k3_status k3_mxfp4_quantize_f32(const float *v, int rows, int cols, uint8_t *nib,
                                uint8_t *sc, k3_stream_t stream);
k3_status k3_mxfp4_quantize_bf16(const uint16_t *v, int rows, int cols,
                                 uint8_t *nib, uint8_t *sc, k3_stream_t stream);
size_t k3_moe_prefill_workspace_bytes(int T, int n_experts, int hidden,
                                      int inter, int k);
k3_status k3_moe_prefill(const uint16_t *X, const double *logits,
                         const float *bias, const uint8_t *const *experts,
                         int n_experts, int hidden, int inter, int k, int T,
                         uint16_t *Y, float *Y_f32, int32_t *idx, float *w,
                         float *h_f32, uint8_t *h_nib, uint8_t *h_sc, void *ws,
                         size_t ws_bytes, k3_stream_t stream);

/* ------------------------------------------------------------------------
 * Shared experts: SwiGLU FFNs with bf16 weights that run on every token and
 * are added to the routed mix ([ZOR] "How does a 2.78-trillion-parameter
 * model fit in 8 GB?": two per layer, in the always-on bf16 set; the pages
 * give neither their width nor how they join the routed output: here any
 * inter_shared (a multiple of 32, <= K3_MAX_INTER) and an unweighted sum).
 *
 * k3_shared_expert_bytes  6 * hidden * inter (0 for unsupported shapes).
 * k3_shared_experts       ys[r] = sum_{s < n_shared} (W_down(s) h[s])[r],
 *                         h[s] = SiLU(W_gate(s) x) * (W_up(s) x). shared: a
 *                         device array of n_shared device pointers, each to a
 *                         blob of gate [inter][hidden], up [inter][hidden],
 *                         down [hidden][inter], bf16 row-major, 16-byte
 *                         aligned. x bf16 [hidden]; h fp32 [n_shared][inter];
 *                         ys fp32 [hidden]. 1 <= n_shared <= K3_MAX_SHARED.
 *                         fp32 accumulation in a fixed order per row.
 * k3_moe_layer_shared     the decode layer of k3_moe_layer_ex with the
 *                         shared experts' ys added to each output row after
 *                         the routed rank-order sum (y_f32 = routed + ys,
 *                         then y = bf16 RNE of it). n_shared may be 0 (then
 *                         the plain layer). Workspace of
 *                         k3_moe_layer_shared_workspace_bytes bytes.
 * ---------------------------------------------------------------------- */
size_t k3_shared_expert_bytes(int hidden, int inter);
k3_status k3_shared_experts(const uint16_t *x, const uint16_t *const *shared,
                            int n_shared, int hidden, int inter, float *h,
                            float *ys, k3_stream_t stream);
size_t k3_moe_layer_shared_workspace_bytes(int n_experts, int hidden, int inter,
                                           int k, int n_shared, int inter_shared);
k3_status k3_moe_layer_shared(const uint16_t *x, const uint16_t *router_w,
                              const uint8_t *const *experts, int n_experts,
                              int hidden, int inter, int k,
                              const uint16_t *const *shared, int n_shared,
                              int inter_shared, uint16_t *y, float *y_f32,
                              int32_t *idx, float *w, double *logits, void *ws,
                              size_t ws_bytes, k3_stream_t stream);

/* Bounded waits, and a way for tests to see them run out. The launches
 * whose workgroups hand data to each other (the decode layer's expert
 * launch behind k3_moe_layer and its peers, and k3_expert_swiglu_ws) poll
 * for each hand-off at most K3_WAIT_LIMIT_DEFAULT times, about a second;
 * if the polls run out the launch still ends, and writes NaN to its fp32
 * output (0x7FC0 to a bf16 one) instead of its result. k3_set_wait_limit sets that number of
 * polls for later launches on the current device: 0 makes every such wait
 * fail at once, so that report can be checked without holding the device
 * for a second. K3_ERR_CONFIG for polls < 0. The value is copied to the device
 * synchronously; a launch already running may use either value. */
#define K3_WAIT_LIMIT_DEFAULT (1 << 20)
k3_status k3_set_wait_limit(int polls);

/* Calibration read for measurements: streams `bytes` (a positive multiple
 * of 16; buf 16-byte aligned, device) once with 16-byte non-temporal loads,
 * one 512-thread workgroup per compute unit. The HBM read rate it reaches is
 * the yardstick the kernels' rates are also reported against. sink: device
 * uint32 [1], written only in the unlikely case the data folds to a fixed
 * value (it keeps the loads from being dropped). */
k3_status k3_hbm_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                            k3_stream_t stream);

/* ------------------------------------------------------------------------
 * Dequantise-then-multiply control: the byte gap the pages price ([SAT]
 * "Reduction one": an expert is 17.55 MB packed and 132 MB as floats; the
 * product waits on bytes). Not on the packed path; it exists to measure it.
 *
 * k3_expert_dense_bytes  12 * hidden * inter (0 for unsupported shapes).
 * k3_expert_dequantize   expert (k3_expert_pack blob, device) -> dense
 *                        (device fp32, k3_expert_dense_bytes): gate
 *                        [inter][hidden], up [inter][hidden], down
 *                        [hidden][inter], row-major, back to back. Weight =
 *                        E2M1(code) * 2^(e-127), exact for exponent bytes
 *                        0..252 (253 and 254 may overflow to inf); groups
 *                        with exponent byte 255 are written as zeros.
 * k3_experts_dense       yp[j] = W_down h[j], h[j] = SiLU(W_gate x) *
 *                        (W_up x) for the dense blob dense_experts[idx[j]],
 *                        j < k: the stages of k3_expert_gate_up and
 *                        k3_expert_down from dense fp32 copies (fp32
 *                        accumulation, fixed order per row). x bf16
 *                        [hidden], h fp32 [k][inter], yp fp32 [k][hidden];
 *                        dense_experts a device pointer table, idx device
 *                        int32 [k] indexing it. Pointers 16-byte aligned.
 * ---------------------------------------------------------------------- */
size_t k3_expert_dense_bytes(int hidden, int inter);
k3_status k3_expert_dequantize(const uint8_t *expert, int hidden, int inter,
                               float *dense, k3_stream_t stream);
k3_status k3_experts_dense(const uint16_t *x, const float *const *dense_experts,
                           const int32_t *idx, int k, int hidden, int inter,
                           float *h, float *yp, k3_stream_t stream);

/* ------------------------------------------------------------------------
 * Expert cache: packed expert blobs (k3_expert_pack layout) in host memory,
 * a fixed number of HBM slots holding the ones in use; the GPU counterpart
 * of the pages' expert LRU that streams experts from NVMe into RAM ([ZOR]
 * "How does a 2.78-trillion-parameter model fit in 8 GB?").
 *
 * A request names experts. Each is a hit (resident, copy finished), an
 * in-flight reuse (its copy was issued and has not finished: the request's
 * stream waits for that copy, none is issued twice) or a miss (copied from
 * its host blob into an empty slot, else into the least recently used slot
 * that is neither pinned nor named by the same request). Copies are
 * asynchronous on the request's stream; keep one stream per cache so that a
 * slot is overwritten only after the kernels queued before it. Host blobs
 * should be pinned (hipHostMalloc) for the copies to be asynchronous.
 * The policy calls are serialised by a lock; k3_moe_layer_cached also uses
 * the cache's one pinned selection buffer, so its calls on one cache must
 * not overlap (one calling thread per cache, as one stream per cache).
 *
 * k3_cache_create     n_slots HBM slots of expert_bytes (a multiple of 256)
 *                     for experts 0..n_experts-1 on the current device,
 *                     plus one all-zero blob and the pointer table
 *                     ((n_slots + 1) * expert_bytes + 8 * n_experts bytes).
 *                     K3_ERR_CONFIG on sizes outside 1 <= n_slots <=
 *                     n_experts <= K3_MAX_EXPERTS; *out is NULL on failure.
 * k3_cache_destroy    frees everything; the caller first synchronises the
 *                     streams that used the cache.
 * k3_cache_set_source host blob of an expert (kept by the caller).
 * k3_cache_pin        pinned experts are never evicted.
 * k3_cache_fetch      makes ids[0..count) (host array) resident; K3_ERR_ARG
 *                     for an id outside [0, n_experts), K3_ERR_CONFIG for a
 *                     missing expert without a source, K3_ERR_MEMORY (and
 *                     nothing changed) if the distinct misses exceed the
 *                     slots that are neither pinned nor already named.
 *                     Calls on one cache are serialised by a lock.
 * k3_cache_table      device array of n_experts pointers (owned by the
 *                     cache): a resident expert's entry points at its slot,
 *                     every other entry at an all-zero blob of the same
 *                     size. Pass it as `experts` to the layer calls on the
 *                     fetch's stream.
 * k3_cache_get_stats, k3_cache_histogram (n_experts counts), k3_cache_trace
 *                     (every requested id in order; *len = full length,
 *                     at most cap copied).
 * k3_cache_replay     runs the same policy on a recorded trace on the host
 *                     alone (requests of request_size ids, every copy taken
 *                     as finished), e.g. to choose a slot count.
 * k3_cache_replay_opt the same replay with the optimal offline victim
 *                     (Belady: the evictable slot whose expert is next used
 *                     farthest ahead; never again is farthest; ties to the
 *                     lowest slot): the bound for an online policy.
 * k3_moe_layer_cached the decode layer for one token through a cache:
 *                     router and top-k on the device, the selection copied
 *                     to the host (this call waits for it), the fetch, then
 *                     the expert launch on the cache's table. Arguments as
 *                     k3_moe_layer_ex; refused while the stream is being
 *                     captured (the host decides the copies).
 * ---------------------------------------------------------------------- */
typedef struct k3_cache_stats {
  uint64_t requests, hits, misses, inflight_reuses, evictions, bytes_copied;
} k3_cache_stats;
typedef struct ExpertCacheImpl *k3_cache_t;

k3_status k3_cache_create(int n_experts, size_t expert_bytes, int n_slots,
                          k3_cache_t *out);
void k3_cache_destroy(k3_cache_t cache);
k3_status k3_cache_set_source(k3_cache_t cache, int expert, const void *host_blob);
k3_status k3_cache_pin(k3_cache_t cache, int expert, int pinned);
k3_status k3_cache_fetch(k3_cache_t cache, const int32_t *ids, int count,
                         k3_stream_t stream);
const uint8_t *const *k3_cache_table(k3_cache_t cache);
k3_status k3_cache_get_stats(k3_cache_t cache, k3_cache_stats *out);
k3_status k3_cache_histogram(k3_cache_t cache, uint64_t *counts);
k3_status k3_cache_trace(k3_cache_t cache, int32_t *buf, size_t cap, size_t *len);
k3_status k3_cache_replay(const int32_t *trace, size_t len, int n_experts,
                          int n_slots, const int32_t *pinned, int n_pinned,
                          int request_size, k3_cache_stats *out);
k3_status k3_cache_replay_opt(const int32_t *trace, size_t len, int n_experts,
                              int n_slots, const int32_t *pinned, int n_pinned,
                              int request_size, k3_cache_stats *out);
/* Batched decode through a cache (as k3_moe_layer_from_logits): top-k of
 * the T tokens, the T*k selection copied to the host (this call waits for
 * it), one fetch of all of it (K3_ERR_MEMORY when its distinct misses
 * exceed the evictable slots), then the resident batched layer on the
 * cache's table, with the same bits. Refused under graph capture. */
k3_status k3_moe_layer_from_logits_cached(const uint16_t *X, const double *logits,
                                          const float *bias, k3_cache_t cache,
                                          int n_experts, int hidden, int inter, int k,
                                          int T, uint16_t *Y, float *Y_f32,
                                          int32_t *idx, float *w, void *ws,
                                          size_t ws_bytes, k3_stream_t stream);
k3_status k3_moe_layer_cached(const uint16_t *x, const uint16_t *router_w,
                              k3_cache_t cache, int n_experts, int hidden,
                              int inter, int k, uint16_t *y, float *y_f32,
                              int32_t *idx, float *w, double *logits, void *ws,
                              size_t ws_bytes, k3_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif
