// C ABI of libk3moe.so: argument validation, workspace carving and the
// launch sequence of each entry point. Every check happens before the first
// launch, so a refused call enqueues nothing (the pages' config reader that
// refuses to guess, [A176] "What byte-identical actually costs"; the up-front
// memory refusal, [A176] "The interesting design decisions").
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>

#include "k3_internal.h"

namespace k3 {

void pack_plain_host(const uint8_t *nib, const uint8_t *sc, int rows, int cols,
                     uint8_t *tiles);
void unpack_plain_host(const uint8_t *tiles, int rows, int cols, uint8_t *nib,
                       uint8_t *sc);
void pack_expert_host(const uint8_t *gn, const uint8_t *gs, const uint8_t *un,
                      const uint8_t *us, const uint8_t *dn, const uint8_t *ds,
                      int hidden, int inter, uint8_t *dst);

namespace {
thread_local char g_err[512];

constexpr int kMaxDim = 1 << 20;  // rows / cols / hidden / inter / T bound
constexpr int kMaxPairs = 1 << 20;  // T*k routing pairs of a batched call

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WsLayout {
  size_t logits, idx, w, h, yp, sync, total;
};

WsLayout ws_layout(int T, int n, int hidden, int inter, int k) {
  WsLayout L;
  size_t off = 0;
  L.logits = off;
  off += align256((size_t)T * n * sizeof(double));
  L.idx = off;
  off += align256((size_t)T * k * sizeof(int32_t));
  L.w = off;
  off += align256((size_t)T * k * sizeof(float));
  L.h = off;
  off += align256((size_t)T * k * inter * sizeof(float));
  L.yp = off;
  off += align256((size_t)T * k * hidden * sizeof(float));
  L.sync = off;
  off += align256((size_t)2 * kMaxSyncGrid * sizeof(uint64_t));
  L.total = off;
  return L;
}

// Per-call values of the layer's arrival slots: unique in the process (a
// counter) and unlikely to equal leftover memory (a random start).
uint64_t next_layer_seq() {
  static std::atomic<uint64_t> seq{[] {
    uint64_t z = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                 ((uint64_t)getpid() << 32);
    z += 0x9E3779B97F4A7C15ull;  // splitmix64 finaliser
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (z ^ (z >> 31)) >> 8;
  }()};
  return seq.fetch_add(1, std::memory_order_relaxed) * 4;
}

// Permutation scratch of T*k pairs (after the caller's counts, offsets,
// pair_token, pair_slot): pair_pos, item_e, item_off, item_cnt, n_items,
// n_bad, and the per-chunk table when the chunks are placed by workgroups of
// their own (chunk_table 0 otherwise).
struct PermWs {
  size_t pair_pos, item_e, item_off, item_cnt, n_items, n_bad, chunk_table, total;
};
PermWs perm_ws(size_t off, int T, int k) {
  PermWs W;
  const size_t a = align256(sizeof(int32_t) * (size_t)T * k);
  W.pair_pos = off;
  W.item_e = W.pair_pos + a;
  W.item_off = W.item_e + a;
  W.item_cnt = W.item_off + a;
  W.n_items = W.item_cnt + a;
  W.n_bad = W.n_items + 256;
  const size_t ct = sizeof(int32_t) * (size_t)perm_chunk_table_ints(T);
  W.chunk_table = ct ? W.n_bad + 256 : 0;
  W.total = W.n_bad + 256 + align256(ct);
  return W;
}

// Batched layer: logits, idx, w, counts, offsets, pair_token, pair_slot,
// the permutation scratch, h [P][inter] (fp32, the one-token path), the bf16
// pieces of h hp [3][P][inter], yp [P][hidden].
struct BatchWs {
  size_t logits, idx, w, counts, offsets, pair_token, pair_slot;
  PermWs perm;
  size_t h, hp, yp, sync, total;
};
BatchWs batch_ws(int T, int n, int hidden, int inter, int k) {
  BatchWs B;
  const long long P = (long long)T * k;
  size_t off = 0;
  B.logits = off;
  off += align256((size_t)T * n * sizeof(double));
  B.idx = off;
  off += align256((size_t)P * sizeof(int32_t));
  B.w = off;
  off += align256((size_t)P * sizeof(float));
  B.counts = off;
  off += align256((size_t)n * sizeof(int32_t));
  B.offsets = off;
  off += align256((size_t)n * sizeof(int32_t));
  B.pair_token = off;
  off += align256((size_t)P * sizeof(int32_t));
  B.pair_slot = off;
  off += align256((size_t)P * sizeof(int32_t));
  B.perm = perm_ws(off, T, k);
  off = B.perm.total;
  B.h = off;
  off += align256((size_t)P * inter * sizeof(float));
  B.hp = off;
  off += align256((size_t)3 * P * inter * sizeof(uint16_t));
  B.yp = off;
  off += align256((size_t)P * hidden * sizeof(float));
  B.sync = off;  // the single-token path's arrival slots (T == 1)
  off += align256((size_t)2 * kMaxSyncGrid * sizeof(uint64_t));
  B.total = off;
  return B;
}

// Prefill: idx, w, counts, offsets, pair_token, pair_slot, permutation
// scratch, quantised x, quantised h, yp [P][hidden] fp32.
struct PrefillWs {
  size_t idx, w, counts, offsets, pair_token, pair_slot;
  PermWs perm;
  size_t xq, xsc, hq, hsc, yp, total;
};
PrefillWs prefill_ws(int T, int n, int hidden, int inter, int k) {
  PrefillWs B;
  const long long P = (long long)T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  B.idx = take((size_t)P * sizeof(int32_t));
  B.w = take((size_t)P * sizeof(float));
  B.counts = take((size_t)n * sizeof(int32_t));
  B.offsets = take((size_t)n * sizeof(int32_t));
  B.pair_token = take((size_t)P * sizeof(int32_t));
  B.pair_slot = take((size_t)P * sizeof(int32_t));
  B.perm = perm_ws(off, T, k);
  off = B.perm.total;
  B.xq = take((size_t)T * hidden / 2);
  B.xsc = take((size_t)T * hidden / 32);
  B.hq = take((size_t)P * inter / 2);
  B.hsc = take((size_t)P * inter / 32);
  B.yp = take((size_t)P * hidden * sizeof(float));
  B.total = off;
  return B;
}

PermOut perm_out(uint8_t *base, const PermWs &W, int32_t *counts,
                 int32_t *offsets, int32_t *pair_token, int32_t *pair_slot) {
  PermOut o;
  o.counts = counts;
  o.offsets = offsets;
  o.pair_token = pair_token;
  o.pair_slot = pair_slot;
  o.pair_pos = reinterpret_cast<int32_t *>(base + W.pair_pos);
  o.item_e = reinterpret_cast<int32_t *>(base + W.item_e);
  o.item_off = reinterpret_cast<int32_t *>(base + W.item_off);
  o.item_cnt = reinterpret_cast<int32_t *>(base + W.item_cnt);
  o.n_items = reinterpret_cast<int32_t *>(base + W.n_items);
  o.n_bad = reinterpret_cast<int32_t *>(base + W.n_bad);
  o.chunk_table = W.chunk_table ? reinterpret_cast<int32_t *>(base + W.chunk_table) : nullptr;
  return o;
}

k3_status fail(k3_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

k3_status device_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return K3_OK;
  return fail(K3_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e,
              hipGetErrorString(e));
}

}  // namespace k3

using namespace k3;

#define K3_NEED_PTR(fn, p)                                                    \
  do {                                                                        \
    if (!(p)) return fail(K3_ERR_ARG, "%s: %s is NULL", fn, #p);              \
    if (!aligned16(p))                                                        \
      return fail(K3_ERR_ARG, "%s: %s is not 16-byte aligned", fn, #p);       \
  } while (0)

#define K3_NEED(fn, cond, ...)                                                \
  do {                                                                        \
    if (!(cond)) return fail(K3_ERR_CONFIG, __VA_ARGS__);                     \
  } while (0)

#define K3_LAUNCH(fn, expr)                                                   \
  do {                                                                        \
    const hipError_t e_ = (expr);                                             \
    if (e_ != hipSuccess) return device_status(e_, fn);                       \
  } while (0)

static k3_status check_mat(const char *fn, int rows, int cols) {
  K3_NEED(fn, rows >= 1 && rows <= kMaxDim, "%s: rows=%d outside [1, %d]", fn,
          rows, kMaxDim);
  K3_NEED(fn, cols >= 32 && cols <= kMaxDim && cols % 32 == 0,
          "%s: cols=%d must be a positive multiple of the group size 32 "
          "(<= %d)",
          fn, cols, kMaxDim);
  return K3_OK;
}

static k3_status check_expert_dims(const char *fn, int hidden, int inter) {
  K3_NEED(fn, hidden >= 32 && hidden <= K3_MAX_HIDDEN && hidden % 32 == 0,
          "%s: hidden=%d must be a positive multiple of 32 (<= %d)", fn,
          hidden, K3_MAX_HIDDEN);
  K3_NEED(fn, inter >= 32 && inter <= K3_MAX_INTER && inter % 32 == 0,
          "%s: inter=%d must be a positive multiple of 32 (<= %d)", fn, inter,
          K3_MAX_INTER);
  return K3_OK;
}

static k3_status check_routing(const char *fn, int T, int n, int k) {
  K3_NEED(fn, T >= 1 && T <= kMaxDim, "%s: T=%d outside [1, %d]", fn, T,
          kMaxDim);
  K3_NEED(fn, n >= 1 && n <= K3_MAX_EXPERTS, "%s: n_experts=%d outside [1, %d]",
          fn, n, K3_MAX_EXPERTS);
  K3_NEED(fn, k >= 1 && k <= n && k <= K3_MAX_TOPK,
          "%s: k=%d outside [1, min(n_experts=%d, %d)]", fn, k, n,
          K3_MAX_TOPK);
  return K3_OK;
}

extern "C" {

const char *k3_strerror(k3_status s) {
  switch (s) {
    case K3_OK: return "ok";
    case K3_ERR_ARG: return "invalid argument (NULL or misaligned pointer)";
    case K3_ERR_CONFIG: return "unsupported or contradictory configuration";
    case K3_ERR_MEMORY:
      return "insufficient memory: the workspace or the cache slots given are smaller than the call needs";
    case K3_ERR_DEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *k3_last_error(void) { return g_err; }

int k3_abi_version(void) { return 1; }

size_t k3_mxfp4_packed_bytes(int rows, int cols) {
  if (check_mat("k3_mxfp4_packed_bytes", rows, cols) != K3_OK) return 0;
  return mat_layout(rows, cols).bytes();
}

k3_status k3_mxfp4_pack_host(const uint8_t *nib, const uint8_t *sc, int rows,
                             int cols, uint8_t *tiles) {
  const char *fn = "k3_mxfp4_pack_host";
  if (!nib || !sc || !tiles) return fail(K3_ERR_ARG, "%s: NULL pointer", fn);
  if (k3_status s = check_mat(fn, rows, cols)) return s;
  pack_plain_host(nib, sc, rows, cols, tiles);
  return K3_OK;
}

k3_status k3_mxfp4_unpack_host(const uint8_t *tiles, int rows, int cols,
                               uint8_t *nib, uint8_t *sc) {
  const char *fn = "k3_mxfp4_unpack_host";
  if (!nib || !sc || !tiles) return fail(K3_ERR_ARG, "%s: NULL pointer", fn);
  if (k3_status s = check_mat(fn, rows, cols)) return s;
  unpack_plain_host(tiles, rows, cols, nib, sc);
  return K3_OK;
}

k3_status k3_mxfp4_pack(const uint8_t *nib_d, const uint8_t *sc_d, int rows,
                        int cols, uint8_t *tiles_d, k3_stream_t stream) {
  const char *fn = "k3_mxfp4_pack";
  K3_NEED_PTR(fn, nib_d);
  if (!sc_d) return fail(K3_ERR_ARG, "%s: sc_d is NULL", fn);
  K3_NEED_PTR(fn, tiles_d);
  if (k3_status s = check_mat(fn, rows, cols)) return s;
  K3_LAUNCH(fn, launch_pack(nib_d, sc_d, rows, cols, tiles_d, stream));
  return K3_OK;
}

k3_status k3_mxfp4_unpack(const uint8_t *tiles_d, int rows, int cols,
                          uint8_t *nib_d, uint8_t *sc_d, k3_stream_t stream) {
  const char *fn = "k3_mxfp4_unpack";
  K3_NEED_PTR(fn, tiles_d);
  K3_NEED_PTR(fn, nib_d);
  if (!sc_d) return fail(K3_ERR_ARG, "%s: sc_d is NULL", fn);
  if (k3_status s = check_mat(fn, rows, cols)) return s;
  K3_LAUNCH(fn, launch_unpack(tiles_d, rows, cols, nib_d, sc_d, stream));
  return K3_OK;
}

size_t k3_expert_packed_bytes(int hidden, int inter) {
  if (check_expert_dims("k3_expert_packed_bytes", hidden, inter) != K3_OK)
    return 0;
  return expert_layout(hidden, inter).bytes();
}

k3_status k3_expert_pack_host(const uint8_t *gate_nib, const uint8_t *gate_sc,
                              const uint8_t *up_nib, const uint8_t *up_sc,
                              const uint8_t *down_nib, const uint8_t *down_sc,
                              int hidden, int inter, uint8_t *expert) {
  const char *fn = "k3_expert_pack_host";
  if (!gate_nib || !gate_sc || !up_nib || !up_sc || !down_nib || !down_sc ||
      !expert)
    return fail(K3_ERR_ARG, "%s: NULL pointer", fn);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  pack_expert_host(gate_nib, gate_sc, up_nib, up_sc, down_nib, down_sc, hidden,
                   inter, expert);
  return K3_OK;
}

k3_status k3_expert_pack(const uint8_t *gate_nib_d, const uint8_t *gate_sc_d,
                         const uint8_t *up_nib_d, const uint8_t *up_sc_d,
                         const uint8_t *down_nib_d, const uint8_t *down_sc_d,
                         int hidden, int inter, uint8_t *expert_d,
                         k3_stream_t stream) {
  const char *fn = "k3_expert_pack";
  K3_NEED_PTR(fn, gate_nib_d);
  K3_NEED_PTR(fn, up_nib_d);
  K3_NEED_PTR(fn, down_nib_d);
  K3_NEED_PTR(fn, expert_d);
  if (!gate_sc_d || !up_sc_d || !down_sc_d)
    return fail(K3_ERR_ARG, "%s: a scale pointer is NULL", fn);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_expert_pack(gate_nib_d, gate_sc_d, up_nib_d, up_sc_d,
                                   down_nib_d, down_sc_d, hidden, inter,
                                   expert_d, stream));
  return K3_OK;
}

static k3_status need_ws(const char *fn, size_t have, size_t need) {
  if (have < need)
    return fail(K3_ERR_MEMORY,
                "%s: workspace of %zu bytes is below the %zu bytes this call "
                "needs (give a larger workspace; no size limit of the path is reached)",
                fn, have, need);
  return K3_OK;
}

k3_status k3_mxfp4_gemv(const float *x, const uint8_t *tiles, int rows,
                        int cols, float *y, k3_stream_t stream) {
  const char *fn = "k3_mxfp4_gemv";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, tiles);
  K3_NEED_PTR(fn, y);
  if (k3_status s = check_mat(fn, rows, cols)) return s;
  K3_LAUNCH(fn, launch_gemv_f32(x, tiles, rows, cols, y, stream));
  return K3_OK;
}

k3_status k3_expert_swiglu(const uint16_t *x, const uint8_t *expert,
                           int hidden, int inter, float *y, float *h,
                           k3_stream_t stream) {
  const char *fn = "k3_expert_swiglu";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, expert);
  K3_NEED_PTR(fn, y);
  K3_NEED_PTR(fn, h);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_gate_up(x, nullptr, nullptr, expert, 1, hidden, inter, h,
                               stream));
  K3_LAUNCH(fn, launch_down(h, nullptr, nullptr, expert, 1, hidden, inter, y,
                            stream));
  return K3_OK;
}

size_t k3_expert_swiglu_workspace_bytes(int hidden, int inter) {
  if (check_expert_dims("k3_expert_swiglu_workspace_bytes", hidden, inter) != K3_OK) return 0;
  return align256(expert_one_workspace_bytes(hidden, inter));
}

k3_status k3_expert_swiglu_ws(const uint16_t *x, const uint8_t *expert, int hidden,
                              int inter, float *y, float *h, void *ws, size_t ws_bytes,
                              k3_stream_t stream) {
  const char *fn = "k3_expert_swiglu_ws";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, expert);
  K3_NEED_PTR(fn, y);
  K3_NEED_PTR(fn, ws);
  if (h && !aligned16(h)) return fail(K3_ERR_ARG, "%s: h is not 16-byte aligned", fn);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  if (k3_status s = need_ws(fn, ws_bytes, k3_expert_swiglu_workspace_bytes(hidden, inter)))
    return s;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (moe_experts_grid() <= (unsigned)kMaxSyncGrid &&
      hipStreamIsCapturing(stream, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone) {
    K3_LAUNCH(fn, launch_expert_one(x, expert, hidden, inter, y, h, ws, next_layer_seq(),
                                    stream));
    return K3_OK;
  }
  // captured (a per-call value would be frozen in the graph): the two stages
  float *hh = h ? h : static_cast<float *>(ws);  // the partial area holds inter floats
  K3_LAUNCH(fn, launch_gate_up(x, nullptr, nullptr, expert, 1, hidden, inter, hh, stream));
  K3_LAUNCH(fn, launch_down(hh, nullptr, nullptr, expert, 1, hidden, inter, y, stream));
  return K3_OK;
}

k3_status k3_expert_gate_up(const uint16_t *x, const uint8_t *const *experts,
                            const int32_t *idx, int k, int hidden, int inter,
                            float *h, k3_stream_t stream) {
  const char *fn = "k3_expert_gate_up";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, h);
  K3_NEED(fn, k >= 1 && k <= K3_MAX_TOPK, "%s: k=%d outside [1, %d]", fn, k,
          K3_MAX_TOPK);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_gate_up(x, experts, idx, nullptr, k, hidden, inter, h,
                               stream));
  return K3_OK;
}

k3_status k3_hbm_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                            k3_stream_t stream) {
  const char *fn = "k3_hbm_read_probe";
  K3_NEED_PTR(fn, buf);
  K3_NEED_PTR(fn, sink);
  K3_NEED(fn, bytes >= 16 && bytes % 16 == 0, "%s: bytes=%zu must be a positive multiple of 16",
          fn, bytes);
  K3_LAUNCH(fn, launch_read_probe(buf, bytes, sink, stream));
  return K3_OK;
}

k3_status k3_set_wait_limit(int polls) {
  const char *fn = "k3_set_wait_limit";
  K3_NEED(fn, polls >= 0, "%s: polls=%d must be >= 0", fn, polls);
  K3_LAUNCH(fn, set_expert_wait_limit(polls));
  K3_LAUNCH(fn, set_expert_one_wait_limit(polls));
  return K3_OK;
}

size_t k3_expert_dense_bytes(int hidden, int inter) {
  if (check_expert_dims("k3_expert_dense_bytes", hidden, inter) != K3_OK) return 0;
  return (size_t)3 * hidden * inter * sizeof(float);
}

k3_status k3_expert_dequantize(const uint8_t *expert, int hidden, int inter,
                               float *dense, k3_stream_t stream) {
  const char *fn = "k3_expert_dequantize";
  K3_NEED_PTR(fn, expert);
  K3_NEED_PTR(fn, dense);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_dequant_expert(expert, hidden, inter, dense, stream));
  return K3_OK;
}

k3_status k3_experts_dense(const uint16_t *x, const float *const *dense_experts,
                           const int32_t *idx, int k, int hidden, int inter,
                           float *h, float *yp, k3_stream_t stream) {
  const char *fn = "k3_experts_dense";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, dense_experts);
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, h);
  K3_NEED_PTR(fn, yp);
  K3_NEED(fn, k >= 1 && k <= K3_MAX_TOPK, "%s: k=%d outside [1, %d]", fn, k,
          K3_MAX_TOPK);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_experts_dense(x, dense_experts, idx, k, hidden, inter, h, yp,
                                     stream));
  return K3_OK;
}

k3_status k3_expert_gate_up_routed(const uint16_t *x, const double *logits,
                                   const uint8_t *const *experts, int n_experts,
                                   int k, int hidden, int inter, float *h,
                                   int32_t *idx, float *w, k3_stream_t stream) {
  const char *fn = "k3_expert_gate_up_routed";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, logits);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, h);
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, w);
  if (k3_status s = check_routing(fn, 1, n_experts, k)) return s;
  K3_NEED(fn, n_experts <= kFusedTopkMaxExperts,
          "%s: n_experts=%d above the %d this call ranks in one wave", fn,
          n_experts, kFusedTopkMaxExperts);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_gate_up_routed(x, logits, experts, n_experts, k, hidden,
                                      inter, h, idx, w, stream));
  return K3_OK;
}

k3_status k3_expert_down(const float *h, const uint8_t *const *experts,
                         const int32_t *idx, int k, int hidden, int inter,
                         float *yp, k3_stream_t stream) {
  const char *fn = "k3_expert_down";
  K3_NEED_PTR(fn, h);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, yp);
  K3_NEED(fn, k >= 1 && k <= K3_MAX_TOPK, "%s: k=%d outside [1, %d]", fn, k,
          K3_MAX_TOPK);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_down(h, experts, idx, nullptr, k, hidden, inter, yp,
                            stream));
  return K3_OK;
}

k3_status k3_moe_combine(const float *yp, const float *w, int k, int hidden,
                         uint16_t *y, float *y_f32, k3_stream_t stream) {
  const char *fn = "k3_moe_combine";
  K3_NEED_PTR(fn, yp);
  K3_NEED_PTR(fn, w);
  if (!y && !y_f32) return fail(K3_ERR_ARG, "%s: y and y_f32 are both NULL", fn);
  if ((y && !aligned16(y)) || (y_f32 && !aligned16(y_f32)))
    return fail(K3_ERR_ARG, "%s: an output is not 16-byte aligned", fn);
  K3_NEED(fn, k >= 1 && k <= K3_MAX_TOPK, "%s: k=%d outside [1, %d]", fn, k,
          K3_MAX_TOPK);
  K3_NEED(fn, hidden >= 1 && hidden <= kMaxDim, "%s: hidden=%d outside [1, %d]",
          fn, hidden, kMaxDim);
  K3_LAUNCH(fn, launch_combine(yp, w, k, hidden, y, y_f32, stream));
  return K3_OK;
}

k3_status k3_router(const uint16_t *x, const uint16_t *router_w, int T,
                    int hidden, int n_experts, double *logits,
                    k3_stream_t stream) {
  const char *fn = "k3_router";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, router_w);
  K3_NEED_PTR(fn, logits);
  K3_NEED(fn, T >= 1 && T <= kMaxDim, "%s: T=%d outside [1, %d]", fn, T,
          kMaxDim);
  K3_NEED(fn, hidden >= 8 && hidden <= kMaxDim && hidden % 8 == 0,
          "%s: hidden=%d must be a positive multiple of 8 (<= %d)", fn, hidden,
          kMaxDim);
  K3_NEED(fn, n_experts >= 1 && n_experts <= K3_MAX_EXPERTS,
          "%s: n_experts=%d outside [1, %d]", fn, n_experts, K3_MAX_EXPERTS);
  K3_LAUNCH(fn, launch_router(x, router_w, T, hidden, n_experts, logits,
                              stream));
  return K3_OK;
}

k3_status k3_router_topk(const double *logits, const float *bias, int T,
                         int n_experts, int k, int32_t *idx, float *w,
                         k3_stream_t stream) {
  const char *fn = "k3_router_topk";
  K3_NEED_PTR(fn, logits);
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, w);
  if (bias && !aligned16(bias))
    return fail(K3_ERR_ARG, "%s: bias is not 16-byte aligned", fn);
  if (k3_status s = check_routing(fn, T, n_experts, k)) return s;
  K3_LAUNCH(fn, launch_topk_f64(logits, bias, T, n_experts, k, idx, w, stream));
  return K3_OK;
}

k3_status k3_router_topk_scaled(const double *logits, const float *bias, int T,
                                int n_experts, int k, double routed_scale,
                                int32_t *idx, float *w, k3_stream_t stream) {
  const char *fn = "k3_router_topk_scaled";
  K3_NEED_PTR(fn, logits);
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, w);
  if (bias && !aligned16(bias))
    return fail(K3_ERR_ARG, "%s: bias is not 16-byte aligned", fn);
  K3_NEED(fn, routed_scale > 0.0 && routed_scale < 1e30,
          "%s: routed_scale=%g is not a positive finite factor", fn, routed_scale);
  if (k3_status s = check_routing(fn, T, n_experts, k)) return s;
  K3_LAUNCH(fn, launch_topk_f64(logits, bias, T, n_experts, k, idx, w, stream,
                                routed_scale));
  return K3_OK;
}

k3_status k3_router_topk_f32(const float *logits, const float *bias, int T,
                             int n_experts, int k, int32_t *idx, float *w,
                             k3_stream_t stream) {
  const char *fn = "k3_router_topk_f32";
  K3_NEED_PTR(fn, logits);
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, w);
  if (bias && !aligned16(bias))
    return fail(K3_ERR_ARG, "%s: bias is not 16-byte aligned", fn);
  if (k3_status s = check_routing(fn, T, n_experts, k)) return s;
  K3_LAUNCH(fn, launch_topk_f32(logits, bias, T, n_experts, k, idx, w, stream));
  return K3_OK;
}

size_t k3_moe_workspace_bytes(int T, int n_experts, int hidden, int inter,
                              int k) {
  if (check_routing("k3_moe_workspace_bytes", T, n_experts, k) != K3_OK ||
      check_expert_dims("k3_moe_workspace_bytes", hidden, inter) != K3_OK)
    return 0;
  return ws_layout(T, n_experts, hidden, inter, k).total;
}

// The layer's launches once its arguments are checked: router, then the
// expert work in one launch (its stages marked by a per-call value; a graph
// being captured would replay one value, so it gets the separate launches,
// as does a selection over more than 1024 experts). `add` (or NULL) is
// added to each output row before the bf16 cast. `sh` (or NULL): the shared
// experts' down stage, whose h an earlier launch wrote; the expert launch
// takes it between its two stages, the separate launches run it first. Its
// sum ys is then what is added.
static k3_status layer_launches(const char *fn, const uint16_t *x,
                                const uint16_t *router_w,
                                const uint8_t *const *experts, int n_experts,
                                int hidden, int inter, int k, uint16_t *y,
                                float *y_f32, int32_t *idx, float *w,
                                double *logits, uint8_t *base, const WsLayout &L,
                                const float *add, hipStream_t stream,
                                bool routed_already = false,
                                const SharedStage *sh = nullptr) {
  double *lg = logits ? logits : reinterpret_cast<double *>(base + L.logits);
  int32_t *ix = idx ? idx : reinterpret_cast<int32_t *>(base + L.idx);
  float *wt = w ? w : reinterpret_cast<float *>(base + L.w);
  float *h = reinterpret_cast<float *>(base + L.h);
  float *yp = reinterpret_cast<float *>(base + L.yp);
  if (!routed_already)
    K3_LAUNCH(fn, launch_router(x, router_w, 1, hidden, n_experts, lg, stream));
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (n_experts <= kFusedTopkMaxExperts &&
      moe_experts_grid() <= (unsigned)kMaxSyncGrid &&
      hipStreamIsCapturing(stream, &cap) == hipSuccess &&
      cap == hipStreamCaptureStatusNone) {
    K3_LAUNCH(fn, launch_moe_experts(x, lg, experts, n_experts, k, hidden,
                                     inter, h, yp,
                                     reinterpret_cast<uint64_t *>(base + L.sync),
                                     next_layer_seq(), ix, wt, y, y_f32, stream, add, sh));
    return K3_OK;
  }
  if (sh) {
    K3_LAUNCH(fn, launch_shared_down(sh->hs, sh->shared, sh->n_shared, hidden, sh->inter,
                                     sh->ys, stream));
    add = sh->ys;
  }
  if (n_experts <= kFusedTopkMaxExperts) {  // top-k inside the gate/up launch
    K3_LAUNCH(fn, launch_gate_up_routed(x, lg, experts, n_experts, k, hidden,
                                        inter, h, ix, wt, stream));
  } else {
    K3_LAUNCH(fn, launch_topk_f64(lg, nullptr, 1, n_experts, k, ix, wt, stream));
    K3_LAUNCH(fn, launch_gate_up(x, experts, ix, nullptr, k, hidden, inter, h,
                                 stream));
  }
  K3_LAUNCH(fn, launch_down(h, experts, ix, nullptr, k, hidden, inter, yp,
                            stream));
  K3_LAUNCH(fn, launch_combine(yp, wt, k, hidden, y, y_f32, stream, add));
  return K3_OK;
}

k3_status k3_moe_layer_ex(const uint16_t *x, const uint16_t *router_w,
                          const uint8_t *const *experts, int n_experts,
                          int hidden, int inter, int k, uint16_t *y,
                          float *y_f32, int32_t *idx, float *w,
                          double *logits, void *ws, size_t ws_bytes,
                          k3_stream_t stream) {
  const char *fn = "k3_moe_layer";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, router_w);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, y);
  K3_NEED_PTR(fn, ws);
  if ((y_f32 && !aligned16(y_f32)) || (idx && !aligned16(idx)) ||
      (w && !aligned16(w)) || (logits && !aligned16(logits)))
    return fail(K3_ERR_ARG, "%s: an optional output is not 16-byte aligned",
                fn);
  if (k3_status s = check_routing(fn, 1, n_experts, k)) return s;
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  const WsLayout L = ws_layout(1, n_experts, hidden, inter, k);
  if (k3_status s = need_ws(fn, ws_bytes, L.total)) return s;
  return layer_launches(fn, x, router_w, experts, n_experts, hidden, inter, k, y,
                        y_f32, idx, w, logits, static_cast<uint8_t *>(ws), L,
                        nullptr, stream);
}

// ---- the decode layer without a caller workspace --------------------------
// For callers that cannot allocate device memory: the layer's scratch (logits,
// selection, h, down partials, arrival slots) lives in this file-scope array,
// one copy per device, held until the process ends. Its device address is
// looked up once per device with that device current; host code passes that
// address, never the array's own name (a host-side stand-in).
static __device__ __align__(256) uint8_t scratch[K3_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
uint8_t *g_scratch_at[kMaxDevices];
}  // namespace

static k3_status scratch_address(const char *fn, uint8_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, fn);
  K3_NEED(fn, dev >= 0 && dev < kMaxDevices, "%s: device %d beyond the %d this library serves",
          fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, fn);
    if (!p) return fail(K3_ERR_DEVICE, "%s: no device address for the static scratch", fn);
    g_scratch_at[dev] = static_cast<uint8_t *>(p);
  }
  *out = g_scratch_at[dev];
  return K3_OK;
}

k3_status k3_moe_layer_noalloc(const uint16_t *x, const uint16_t *router_w,
                               const uint8_t *const *experts, int n_experts,
                               int hidden, int inter, int k, uint16_t *y,
                               float *y_f32, int32_t *idx, float *w,
                               double *logits, k3_stream_t stream) {
  const char *fn = "k3_moe_layer_noalloc";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, router_w);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, y);
  if ((y_f32 && !aligned16(y_f32)) || (idx && !aligned16(idx)) ||
      (w && !aligned16(w)) || (logits && !aligned16(logits)))
    return fail(K3_ERR_ARG, "%s: an optional output is not 16-byte aligned",
                fn);
  if (k3_status s = check_routing(fn, 1, n_experts, k)) return s;
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  const WsLayout L = ws_layout(1, n_experts, hidden, inter, k);
  if (L.total > (size_t)K3_NOALLOC_SCRATCH_BYTES)
    return fail(K3_ERR_MEMORY,
                "%s: this shape needs %zu bytes of scratch, above the %zu-byte "
                "static scratch of the call (use k3_moe_layer_ex with a workspace)",
                fn, L.total, (size_t)K3_NOALLOC_SCRATCH_BYTES);
  uint8_t *base = nullptr;
  if (k3_status s = scratch_address(fn, &base)) return s;
  return layer_launches(fn, x, router_w, experts, n_experts, hidden, inter, k, y,
                        y_f32, idx, w, logits, base, L, nullptr, stream);
}

size_t k3_shared_expert_bytes(int hidden, int inter) {
  if (check_expert_dims("k3_shared_expert_bytes", hidden, inter) != K3_OK) return 0;
  return (size_t)3 * hidden * inter * sizeof(uint16_t);
}

k3_status k3_shared_experts(const uint16_t *x, const uint16_t *const *shared,
                            int n_shared, int hidden, int inter, float *h,
                            float *ys, k3_stream_t stream) {
  const char *fn = "k3_shared_experts";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, shared);
  K3_NEED_PTR(fn, h);
  K3_NEED_PTR(fn, ys);
  K3_NEED(fn, n_shared >= 1 && n_shared <= K3_MAX_SHARED,
          "%s: n_shared=%d outside [1, %d]", fn, n_shared, K3_MAX_SHARED);
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_LAUNCH(fn, launch_shared_experts(x, shared, n_shared, hidden, inter, h, ys, stream));
  return K3_OK;
}

// Workspace of k3_moe_layer_shared: the layer's, then h of the shared
// experts and their summed output.
struct SharedWs {
  WsLayout L;
  size_t hs, ys, total;
};
static SharedWs shared_ws(int n, int hidden, int inter, int k, int n_shared,
                          int inter_shared) {
  SharedWs S;
  S.L = ws_layout(1, n, hidden, inter, k);
  size_t off = S.L.total;
  S.hs = off;
  off += align256((size_t)n_shared * inter_shared * sizeof(float));
  S.ys = off;
  off += align256((size_t)hidden * sizeof(float));
  S.total = off;
  return S;
}

size_t k3_moe_layer_shared_workspace_bytes(int n_experts, int hidden, int inter,
                                           int k, int n_shared, int inter_shared) {
  if (n_experts < 1 || k < 1 || n_shared < 0 || n_shared > K3_MAX_SHARED) return 0;
  if (check_expert_dims("k3_moe_layer_shared_workspace_bytes", hidden, inter) != K3_OK)
    return 0;
  if (n_shared > 0 &&
      check_expert_dims("k3_moe_layer_shared_workspace_bytes", hidden, inter_shared) != K3_OK)
    return 0;
  return shared_ws(n_experts, hidden, inter, k, n_shared, inter_shared).total;
}

k3_status k3_moe_layer_shared(const uint16_t *x, const uint16_t *router_w,
                              const uint8_t *const *experts, int n_experts,
                              int hidden, int inter, int k,
                              const uint16_t *const *shared, int n_shared,
                              int inter_shared, uint16_t *y, float *y_f32,
                              int32_t *idx, float *w, double *logits, void *ws,
                              size_t ws_bytes, k3_stream_t stream) {
  const char *fn = "k3_moe_layer_shared";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, router_w);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, y);
  K3_NEED_PTR(fn, ws);
  if ((y_f32 && !aligned16(y_f32)) || (idx && !aligned16(idx)) ||
      (w && !aligned16(w)) || (logits && !aligned16(logits)))
    return fail(K3_ERR_ARG, "%s: an optional output is not 16-byte aligned",
                fn);
  K3_NEED(fn, n_shared >= 0 && n_shared <= K3_MAX_SHARED,
          "%s: n_shared=%d outside [0, %d]", fn, n_shared, K3_MAX_SHARED);
  if (n_shared > 0) {
    K3_NEED_PTR(fn, shared);
    if (k3_status s = check_expert_dims(fn, hidden, inter_shared)) return s;
  }
  if (k3_status s = check_routing(fn, 1, n_experts, k)) return s;
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  const SharedWs S = shared_ws(n_experts, hidden, inter, k, n_shared, inter_shared);
  if (k3_status s = need_ws(fn, ws_bytes, S.total)) return s;
  uint8_t *base = static_cast<uint8_t *>(ws);
  if (n_shared == 0)
    return layer_launches(fn, x, router_w, experts, n_experts, hidden, inter, k, y,
                          y_f32, idx, w, logits, base, S.L, nullptr, stream);
  // The router rows and the shared experts' gate/up rows in one launch, then
  // the expert work with the shared down stage (its sum ys is added to each
  // output row).
  float *ys = reinterpret_cast<float *>(base + S.ys);
  float *hs = reinterpret_cast<float *>(base + S.hs);
  double *lg = logits ? logits : reinterpret_cast<double *>(base + S.L.logits);
  K3_LAUNCH(fn, launch_router_shared(x, router_w, hidden, n_experts, lg, shared, n_shared,
                                     inter_shared, hs, stream));
  const SharedStage sh = {hs, shared, n_shared, inter_shared, ys};
  return layer_launches(fn, x, router_w, experts, n_experts, hidden, inter, k, y, y_f32,
                        idx, w, lg, base, S.L, nullptr, stream, true, &sh);
}

k3_status k3_moe_layer_cached(const uint16_t *x, const uint16_t *router_w,
                              k3_cache_t cache, int n_experts, int hidden,
                              int inter, int k, uint16_t *y, float *y_f32,
                              int32_t *idx, float *w, double *logits, void *ws,
                              size_t ws_bytes, k3_stream_t stream) {
  const char *fn = "k3_moe_layer_cached";
  K3_NEED_PTR(fn, x);
  K3_NEED_PTR(fn, router_w);
  K3_NEED_PTR(fn, y);
  K3_NEED_PTR(fn, ws);
  if (!cache) return fail(K3_ERR_ARG, "%s: cache is NULL", fn);
  if ((y_f32 && !aligned16(y_f32)) || (idx && !aligned16(idx)) ||
      (w && !aligned16(w)) || (logits && !aligned16(logits)))
    return fail(K3_ERR_ARG, "%s: an optional output is not 16-byte aligned", fn);
  if (k3_status s = check_routing(fn, 1, n_experts, k)) return s;
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  K3_NEED(fn, n_experts <= kFusedTopkMaxExperts,
          "%s: n_experts=%d above the %d the expert launch ranks", fn, n_experts,
          kFusedTopkMaxExperts);
  K3_NEED(fn, moe_experts_grid() <= (unsigned)kMaxSyncGrid,
          "%s: %u compute units exceed the %d arrival slots", fn,
          moe_experts_grid(), kMaxSyncGrid);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  K3_NEED(fn, hipStreamIsCapturing(stream, &cap) == hipSuccess &&
                  cap == hipStreamCaptureStatusNone,
          "%s: cannot be captured: the host chooses the copies per token", fn);
  const WsLayout L = ws_layout(1, n_experts, hidden, inter, k);
  if (k3_status s = need_ws(fn, ws_bytes, L.total)) return s;
  uint8_t *base = static_cast<uint8_t *>(ws);
  double *lg = logits ? logits : reinterpret_cast<double *>(base + L.logits);
  int32_t *ix = idx ? idx : reinterpret_cast<int32_t *>(base + L.idx);
  float *wt = w ? w : reinterpret_cast<float *>(base + L.w);
  float *h = reinterpret_cast<float *>(base + L.h);
  float *yp = reinterpret_cast<float *>(base + L.yp);
  int32_t *sel = cache_selection_buffer(cache, (size_t)k);
  if (!sel) return fail(K3_ERR_MEMORY, "%s: pinned selection buffer", fn);
  // the token's selection decides the copies: router and top-k, then wait
  K3_LAUNCH(fn, launch_router(x, router_w, 1, hidden, n_experts, lg, stream));
  K3_LAUNCH(fn, launch_topk_f64(lg, nullptr, 1, n_experts, k, ix, wt, stream));
  K3_LAUNCH(fn, hipMemcpyAsync(sel, ix, sizeof(int32_t) * k, hipMemcpyDeviceToHost,
                               stream));
  K3_LAUNCH(fn, hipStreamSynchronize(stream));
  if (k3_status s = k3_cache_fetch(cache, sel, k, stream)) return s;
  // the expert launch ranks the same logits again and reads the cache's
  // table, which holds every expert of this selection
  K3_LAUNCH(fn, launch_moe_experts(x, lg, k3_cache_table(cache), n_experts, k,
                                   hidden, inter, h, yp,
                                   reinterpret_cast<uint64_t *>(base + L.sync),
                                   next_layer_seq(), ix, wt, y, y_f32, stream));
  return K3_OK;
}

k3_status k3_moe_layer(const uint16_t *x, const uint16_t *router_w,
                       const uint8_t *const *experts, int n_experts,
                       int hidden, int inter, int k, uint16_t *y, void *ws,
                       size_t ws_bytes, k3_stream_t stream) {
  return k3_moe_layer_ex(x, router_w, experts, n_experts, hidden, inter, k, y,
                         nullptr, nullptr, nullptr, nullptr, ws, ws_bytes,
                         stream);
}

/* ---- batched decode ---------------------------------------------------- */

static k3_status check_batch(const char *fn, int T, int n, int k) {
  if (k3_status s = check_routing(fn, T, n, k)) return s;
  K3_NEED(fn, (long long)T * k <= kMaxPairs,
          "%s: T*k=%lld routing pairs above %d", fn, (long long)T * k, kMaxPairs);
  return K3_OK;
}

size_t k3_moe_permute_workspace_bytes(int T, int k) {
  if (T < 1 || k < 1 || k > K3_MAX_TOPK || (long long)T * k > kMaxPairs) return 0;
  return perm_ws(0, T, k).total;
}

k3_status k3_moe_permute(const int32_t *idx, int T, int k, int n_experts,
                         int32_t *counts, int32_t *offsets, int32_t *pair_token,
                         int32_t *pair_slot, void *ws, size_t ws_bytes,
                         k3_stream_t stream) {
  const char *fn = "k3_moe_permute";
  K3_NEED_PTR(fn, idx);
  K3_NEED_PTR(fn, counts);
  K3_NEED_PTR(fn, offsets);
  K3_NEED_PTR(fn, pair_token);
  K3_NEED_PTR(fn, pair_slot);
  K3_NEED_PTR(fn, ws);
  K3_NEED(fn, n_experts >= 1 && n_experts <= K3_MAX_EXPERTS,
          "%s: n_experts=%d outside [1, %d]", fn, n_experts, K3_MAX_EXPERTS);
  K3_NEED(fn, T >= 1 && k >= 1 && k <= K3_MAX_TOPK && (long long)T * k <= kMaxPairs,
          "%s: T=%d k=%d outside T >= 1, 1 <= k <= %d, T*k <= %d", fn, T, k,
          K3_MAX_TOPK, kMaxPairs);
  const PermWs W = perm_ws(0, T, k);
  if (k3_status s = need_ws(fn, ws_bytes, W.total)) return s;
  uint8_t *base = static_cast<uint8_t *>(ws);
  K3_LAUNCH(fn, launch_permute(idx, T, k, n_experts,
                               perm_out(base, W, counts, offsets, pair_token,
                                        pair_slot),
                               gate_up_mfma_tok(), gate_up_mfma_tok(), stream));
  return K3_OK;
}

size_t k3_moe_batched_workspace_bytes(int T, int n_experts, int hidden,
                                      int inter, int k) {
  if (check_batch("k3_moe_batched_workspace_bytes", T, n_experts, k) != K3_OK ||
      check_expert_dims("k3_moe_batched_workspace_bytes", hidden, inter) != K3_OK)
    return 0;
  return batch_ws(T, n_experts, hidden, inter, k).total;
}

static k3_status batched_common(const char *fn, const uint16_t *X,
                                const uint16_t *router_w, const double *logits,
                                const float *bias,
                                const uint8_t *const *experts, int n_experts,
                                int hidden, int inter, int k, int T,
                                uint16_t *Y, float *Y_f32, int32_t *idx,
                                float *w, void *ws, size_t ws_bytes,
                                k3_stream_t stream) {
  K3_NEED_PTR(fn, X);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, ws);
  if (!Y && !Y_f32) return fail(K3_ERR_ARG, "%s: Y and Y_f32 are both NULL", fn);
  if ((Y && !aligned16(Y)) || (Y_f32 && !aligned16(Y_f32)) ||
      (idx && !aligned16(idx)) || (w && !aligned16(w)) ||
      (bias && !aligned16(bias)))
    return fail(K3_ERR_ARG, "%s: an optional argument is not 16-byte aligned",
                fn);
  if (k3_status s = check_batch(fn, T, n_experts, k)) return s;
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  const BatchWs B = batch_ws(T, n_experts, hidden, inter, k);
  if (k3_status s = need_ws(fn, ws_bytes, B.total)) return s;
  uint8_t *base = static_cast<uint8_t *>(ws);
  double *lg = reinterpret_cast<double *>(base + B.logits);
  int32_t *ix = idx ? idx : reinterpret_cast<int32_t *>(base + B.idx);
  float *wt = w ? w : reinterpret_cast<float *>(base + B.w);
  const PermOut o = perm_out(base, B.perm,
                             reinterpret_cast<int32_t *>(base + B.counts),
                             reinterpret_cast<int32_t *>(base + B.offsets),
                             reinterpret_cast<int32_t *>(base + B.pair_token),
                             reinterpret_cast<int32_t *>(base + B.pair_slot));
  float *h = reinterpret_cast<float *>(base + B.h);
  float *yp = reinterpret_cast<float *>(base + B.yp);
  if (router_w) {
    K3_LAUNCH(fn, launch_router(X, router_w, T, hidden, n_experts, lg, stream));
    logits = lg;
  }
  // One token without a routing bias: the single-token decode layer's expert
  // launch (top-k, gate/up, down, combine; as k3_moe_layer after its router).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (T == 1 && !bias && n_experts <= kFusedTopkMaxExperts &&
      moe_experts_grid() <= (unsigned)kMaxSyncGrid &&
      hipStreamIsCapturing(stream, &cap) == hipSuccess &&
      cap == hipStreamCaptureStatusNone) {
    K3_LAUNCH(fn, launch_moe_experts(X, logits, experts, n_experts, k, hidden,
                                     inter, h, yp,
                                     reinterpret_cast<uint64_t *>(base + B.sync),
                                     next_layer_seq(), ix, wt, Y, Y_f32, stream));
    return K3_OK;
  }
  K3_LAUNCH(fn, launch_topk_f64(logits, bias, T, n_experts, k, ix, wt, stream));
  K3_LAUNCH(fn, launch_permute(ix, T, k, n_experts, o, gate_up_mfma_tok(), down_mfma_pack_tok(),
                               stream));
  const long long P = (long long)T * k;
  const int max_items = (int)(std::min<long long>(n_experts, P) + P / gate_up_mfma_tok() + 1);
  uint16_t *hp = reinterpret_cast<uint16_t *>(base + B.hp);
  K3_LAUNCH(fn, launch_gate_up_mfma(X, experts, o, max_items, P, hidden, inter, hp, stream));
  K3_LAUNCH(fn, launch_down_mfma(hp, experts, o, max_items, P, hidden, inter, yp, stream));
  K3_LAUNCH(fn, launch_combine_batched(yp, wt, o.pair_pos, T, k, hidden, Y,
                                       Y_f32, stream));
  return K3_OK;
}

k3_status k3_moe_layer_from_logits(const uint16_t *X, const double *logits,
                                   const float *bias,
                                   const uint8_t *const *experts,
                                   int n_experts, int hidden, int inter, int k,
                                   int T, uint16_t *Y, float *Y_f32,
                                   int32_t *idx, float *w, void *ws,
                                   size_t ws_bytes, k3_stream_t stream) {
  const char *fn = "k3_moe_layer_from_logits";
  K3_NEED_PTR(fn, logits);
  return batched_common(fn, X, nullptr, logits, bias, experts, n_experts, hidden,
                        inter, k, T, Y, Y_f32, idx, w, ws, ws_bytes, stream);
}

k3_status k3_moe_layer_from_logits_cached(const uint16_t *X, const double *logits,
                                          const float *bias, k3_cache_t cache,
                                          int n_experts, int hidden, int inter, int k,
                                          int T, uint16_t *Y, float *Y_f32,
                                          int32_t *idx, float *w, void *ws,
                                          size_t ws_bytes, k3_stream_t stream) {
  const char *fn = "k3_moe_layer_from_logits_cached";
  K3_NEED_PTR(fn, logits);
  K3_NEED_PTR(fn, ws);
  if (!cache) return fail(K3_ERR_ARG, "%s: cache is NULL", fn);
  if (bias && !aligned16(bias)) return fail(K3_ERR_ARG, "%s: bias is not 16-byte aligned", fn);
  if (k3_status s = check_batch(fn, T, n_experts, k)) return s;
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  const BatchWs B = batch_ws(T, n_experts, hidden, inter, k);
  if (k3_status s = need_ws(fn, ws_bytes, B.total)) return s;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  K3_NEED(fn, hipStreamIsCapturing(stream, &cap) == hipSuccess &&
                  cap == hipStreamCaptureStatusNone,
          "%s: cannot be captured: the host chooses the copies per batch", fn);
  const size_t P = (size_t)T * k;
  int32_t *sel = cache_selection_buffer(cache, P);
  if (!sel) return fail(K3_ERR_MEMORY, "%s: pinned selection buffer of %zu ints", fn, P);
  // the batch's selection decides the copies: top-k, then wait for it
  uint8_t *base = static_cast<uint8_t *>(ws);
  int32_t *ix = reinterpret_cast<int32_t *>(base + B.idx);
  float *wt = reinterpret_cast<float *>(base + B.w);
  K3_LAUNCH(fn, launch_topk_f64(logits, bias, T, n_experts, k, ix, wt, stream));
  K3_LAUNCH(fn, hipMemcpyAsync(sel, ix, sizeof(int32_t) * P, hipMemcpyDeviceToHost, stream));
  K3_LAUNCH(fn, hipStreamSynchronize(stream));
  if (k3_status s = k3_cache_fetch(cache, sel, (int)P, stream)) return s;
  // then exactly the resident batched layer, reading the cache's table
  return batched_common(fn, X, nullptr, logits, bias, k3_cache_table(cache), n_experts,
                        hidden, inter, k, T, Y, Y_f32, idx, w, ws, ws_bytes, stream);
}

k3_status k3_moe_layer_batched(const uint16_t *X, const uint16_t *router_w,
                               const uint8_t *const *experts, int n_experts,
                               int hidden, int inter, int k, int T, uint16_t *Y,
                               float *Y_f32, int32_t *idx, float *w, void *ws,
                               size_t ws_bytes, k3_stream_t stream) {
  const char *fn = "k3_moe_layer_batched";
  K3_NEED_PTR(fn, router_w);
  K3_NEED(fn, hidden % 8 == 0, "%s: hidden=%d must be a multiple of 8", fn, hidden);
  return batched_common(fn, X, router_w, nullptr, nullptr, experts, n_experts,
                        hidden, inter, k, T, Y, Y_f32, idx, w, ws, ws_bytes,
                        stream);
}

/* ---- prefill ------------------------------------------------------------ */

static k3_status check_quant(const char *fn, long long rows, int cols) {
  K3_NEED(fn, rows >= 1 && rows <= (1ll << 31), "%s: rows=%lld outside [1, 2^31]", fn,
          rows);
  K3_NEED(fn, cols >= 32 && cols <= kMaxDim && cols % 32 == 0,
          "%s: cols=%d must be a positive multiple of 32 (<= %d)", fn, cols, kMaxDim);
  return K3_OK;
}

k3_status k3_mxfp4_quantize_f32(const float *v, int rows, int cols, uint8_t *nib,
                                uint8_t *sc, k3_stream_t stream) {
  const char *fn = "k3_mxfp4_quantize_f32";
  K3_NEED_PTR(fn, v);
  K3_NEED_PTR(fn, nib);
  if (!sc) return fail(K3_ERR_ARG, "%s: sc is NULL", fn);
  if (k3_status s = check_quant(fn, rows, cols)) return s;
  K3_LAUNCH(fn, launch_quant_f32(v, rows, cols, nib, sc, stream));
  return K3_OK;
}

k3_status k3_mxfp4_quantize_bf16(const uint16_t *v, int rows, int cols,
                                 uint8_t *nib, uint8_t *sc, k3_stream_t stream) {
  const char *fn = "k3_mxfp4_quantize_bf16";
  K3_NEED_PTR(fn, v);
  K3_NEED_PTR(fn, nib);
  if (!sc) return fail(K3_ERR_ARG, "%s: sc is NULL", fn);
  if (k3_status s = check_quant(fn, rows, cols)) return s;
  K3_LAUNCH(fn, launch_quant_bf16(v, rows, cols, nib, sc, stream));
  return K3_OK;
}

size_t k3_moe_prefill_workspace_bytes(int T, int n_experts, int hidden,
                                      int inter, int k) {
  if (check_batch("k3_moe_prefill_workspace_bytes", T, n_experts, k) != K3_OK ||
      check_expert_dims("k3_moe_prefill_workspace_bytes", hidden, inter) != K3_OK)
    return 0;
  return prefill_ws(T, n_experts, hidden, inter, k).total;
}

k3_status k3_moe_prefill(const uint16_t *X, const double *logits,
                         const float *bias, const uint8_t *const *experts,
                         int n_experts, int hidden, int inter, int k, int T,
                         uint16_t *Y, float *Y_f32, int32_t *idx, float *w,
                         float *h_f32, uint8_t *h_nib, uint8_t *h_sc, void *ws,
                         size_t ws_bytes, k3_stream_t stream) {
  const char *fn = "k3_moe_prefill";
  K3_NEED_PTR(fn, X);
  K3_NEED_PTR(fn, logits);
  K3_NEED_PTR(fn, experts);
  K3_NEED_PTR(fn, ws);
  if (!Y && !Y_f32) return fail(K3_ERR_ARG, "%s: Y and Y_f32 are both NULL", fn);
  if ((Y && !aligned16(Y)) || (Y_f32 && !aligned16(Y_f32)) ||
      (idx && !aligned16(idx)) || (w && !aligned16(w)) ||
      (bias && !aligned16(bias)) || (h_f32 && !aligned16(h_f32)) ||
      (h_nib && !aligned16(h_nib)))
    return fail(K3_ERR_ARG, "%s: an optional argument is not 16-byte aligned",
                fn);
  if ((h_nib == nullptr) != (h_sc == nullptr))
    return fail(K3_ERR_ARG, "%s: h_nib and h_sc must be given together", fn);
  if (k3_status s = check_batch(fn, T, n_experts, k)) return s;
  if (k3_status s = check_expert_dims(fn, hidden, inter)) return s;
  const PrefillWs B = prefill_ws(T, n_experts, hidden, inter, k);
  if (k3_status s = need_ws(fn, ws_bytes, B.total)) return s;
  uint8_t *base = static_cast<uint8_t *>(ws);
  int32_t *ix = idx ? idx : reinterpret_cast<int32_t *>(base + B.idx);
  float *wt = w ? w : reinterpret_cast<float *>(base + B.w);
  const PermOut o = perm_out(base, B.perm,
                             reinterpret_cast<int32_t *>(base + B.counts),
                             reinterpret_cast<int32_t *>(base + B.offsets),
                             reinterpret_cast<int32_t *>(base + B.pair_token),
                             reinterpret_cast<int32_t *>(base + B.pair_slot));
  uint8_t *hq = h_nib ? h_nib : base + B.hq;
  uint8_t *hsc = h_sc ? h_sc : base + B.hsc;
  const long long P = (long long)T * k;
  const int max_items =
      (int)(std::min<long long>(n_experts, P) + P / prefill_tok_batch() + 1);
  K3_LAUNCH(fn, launch_topk_f64(logits, bias, T, n_experts, k, ix, wt, stream));
  K3_LAUNCH(fn, launch_permute(ix, T, k, n_experts, o, prefill_tok_batch(), prefill_tok_batch(),
                               stream));
  K3_LAUNCH(fn, launch_quant_bf16(X, T, hidden, base + B.xq, base + B.xsc, stream));
  K3_LAUNCH(fn, launch_prefill_gate_up(base + B.xq, base + B.xsc, experts, o,
                                       max_items, hidden, inter, hq, hsc, h_f32,
                                       stream));
  float *yp = reinterpret_cast<float *>(base + B.yp);
  K3_LAUNCH(fn, launch_prefill_down(hq, hsc, experts, o, max_items, hidden,
                                    inter, yp, stream));
  K3_LAUNCH(fn, launch_combine_batched(yp, wt, o.pair_pos, T, k, hidden, Y,
                                       Y_f32, stream));
  return K3_OK;
}

}  // extern "C"
