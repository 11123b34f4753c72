// Internal declarations of the k3moe library (gfx950 / HIP).
//
// Tile layout of an MXFP4 matrix (the layout the kernels read; see
// include/k3moe.h for the byte-level definition): 64-row tiles, each tile a
// sequence of G4 quad blocks of 4352 bytes: [4 groups][64 lanes][16 B] of
// packed codes then [64 lanes][4 B] of the quad's exponent bytes. One lane
// owns one row; a wave's load of group g is one contiguous KiB, a wave walks
// one contiguous stream, and every quad of groups is whole. Padding (groups
// past G, rows past the matrix) is zero codes with exponent byte 0.
#pragma once

#include <hip/hip_runtime.h>

#include <functional>
#include <stddef.h>
#include <stdint.h>

#include "k3moe.h"

namespace k3 {

constexpr int kTileRows = 64;   // rows per tile = lanes per wave
constexpr int kGroup = 32;      // weights per exponent byte
constexpr int kGroupBytes = 16; // packed bytes per group
constexpr int kQuadBytes = 4352;  // 4 groups x 64 lanes x 16 B + 64 x 4 B

// Byte offsets inside a tile: codes of group g of tile row r (lane r), and
// the exponent byte of group g of tile row r.
__host__ __device__ inline size_t code_offset(int g, int r) {
  return (size_t)kQuadBytes * (g >> 2) + (size_t)1024 * (g & 3) + 16 * r;
}
__host__ __device__ inline size_t scale_offset(int g, int r) {
  return (size_t)kQuadBytes * (g >> 2) + 4096 + 4 * r + (g & 3);
}

struct MatLayout {
  int rows, cols, G, G4, ntiles;
  size_t tile_bytes;  // G4 quad blocks of 4096 code + 256 exponent bytes
  __host__ __device__ size_t bytes() const { return (size_t)ntiles * tile_bytes; }
};

__host__ __device__ inline MatLayout mat_layout(int rows, int cols) {
  MatLayout m;
  m.rows = rows;
  m.cols = cols;
  m.G = cols / kGroup;
  m.G4 = (m.G + 3) / 4;
  m.ntiles = (rows + kTileRows - 1) / kTileRows;
  m.tile_bytes = (size_t)kQuadBytes * m.G4;
  return m;
}

// Expert blob: gate/up region (2*inter virtual rows, 32 gate + 32 up rows per
// tile) followed by the down region (hidden x inter).
struct ExpertLayout {
  MatLayout gu;    // virtual: rows = 64 * ntiles_gu, cols = hidden
  MatLayout down;  // rows = hidden, cols = inter
  int inter, hidden;
  size_t down_offset;
  __host__ __device__ size_t bytes() const { return down_offset + down.bytes(); }
};

__host__ __device__ inline ExpertLayout expert_layout(int hidden, int inter) {
  ExpertLayout e;
  e.hidden = hidden;
  e.inter = inter;
  const int ntiles = (inter + 31) / 32;
  e.gu = mat_layout(ntiles * kTileRows, hidden);
  e.down = mat_layout(hidden, inter);
  e.down_offset = e.gu.bytes();
  return e;
}

// Which canonical (matrix, row) a gate/up tile lane holds: lanes 0..31 the
// gate rows 32t.., lanes 32..63 the up rows 32t...
__host__ __device__ inline void gu_lane_row(int t, int lane, int *is_up,
                                            int *row) {
  *is_up = lane >> 5;
  *row = 32 * t + (lane & 31);
}

// ---- host-side helpers (k3_abi.hip) ----
// Compute units of the current device (cached per device).
int num_cus();
void set_error(const char *fmt, ...);
k3_status device_status(hipError_t e, const char *what);

// ---- launchers (each returns hipSuccess or the launch error) ----
hipError_t launch_pack(const uint8_t *nib, const uint8_t *sc, int rows,
                       int cols, uint8_t *tiles, hipStream_t s);
hipError_t launch_unpack(const uint8_t *tiles, int rows, int cols,
                         uint8_t *nib, uint8_t *sc, hipStream_t s);
hipError_t launch_expert_pack(const uint8_t *gn, const uint8_t *gs,
                              const uint8_t *un, const uint8_t *us,
                              const uint8_t *dn, const uint8_t *ds, int hidden,
                              int inter, uint8_t *dst, hipStream_t s);
hipError_t launch_gemv_f32(const float *x, const uint8_t *tiles, int rows,
                           int cols, float *y, hipStream_t s);
// Gate/up + SwiGLU over `nslots` experts: slot j uses expert experts[idx[j]]
// (or `single` when experts == nullptr); h[j][inter].
hipError_t launch_gate_up(const uint16_t *x, const uint8_t *const *experts,
                          const int32_t *idx, const uint8_t *single,
                          int nslots, int hidden, int inter, float *h,
                          hipStream_t s);
// Down projection: yp[j][hidden] = W_down(e_j) h[j].
hipError_t launch_down(const float *h, const uint8_t *const *experts,
                       const int32_t *idx, const uint8_t *single, int nslots,
                       int hidden, int inter, float *yp, hipStream_t s);
// Batched decode (k3_batched.hip). Permutation outputs, all device arrays:
// counts/offsets [n], pair_token/pair_slot/pair_pos and the work items
// item_e/item_off/item_cnt [T*k], n_items and n_bad [1].
struct PermOut {
  int32_t *counts, *offsets, *pair_token, *pair_slot, *pair_pos;
  int32_t *item_e, *item_off, *item_cnt, *n_items, *n_bad;
  int32_t *chunk_table;  // perm_chunk_table_ints(T) ints, or null: one workgroup does it all
};
// Scratch of the permutation's per-chunk counts when its chunks of 64 tokens
// go to workgroups of their own (0: one workgroup places them all).
int perm_chunk_table_ints(int T);
// Work items of at most item_tok pairs of one expert; those of more than
// pack_tok pairs come first (n_items[1] of them), then the others
// (n_items[0] in all). pack_tok >= item_tok keeps plain expert order.
hipError_t launch_permute(const int32_t *idx, int T, int k, int n,
                          const PermOut &o, int item_tok, int pack_tok, hipStream_t s);
// Batched gate/up and down on the matrix unit, over items of at most
// gate_up_mfma_tok() tokens; X 16-byte aligned. hp: the three bf16 pieces
// of h, [3][P][inter]; yp [P][hidden] fp32.
int gate_up_mfma_tok();
int down_mfma_pack_tok();  // items of at most this many pairs take the packed down launch
hipError_t launch_gate_up_mfma(const uint16_t *X, const uint8_t *const *experts,
                               const PermOut &o, int max_items, long long P, int hidden,
                               int inter, uint16_t *hp, hipStream_t s);
hipError_t launch_down_mfma(const uint16_t *hp, const uint8_t *const *experts, const PermOut &o,
                            int max_items, long long P, int hidden, int inter, float *yp,
                            hipStream_t s);
hipError_t launch_combine_batched(const float *yp, const float *w,
                                  const int32_t *pair_pos, int T, int k,
                                  int hidden, uint16_t *Y, float *Y32,
                                  hipStream_t s);
// Prefill (k3_prefill.hip): MXFP4 quantiser and the FP4 x FP4 grouped GEMMs.
int prefill_tok_batch();
hipError_t launch_quant_bf16(const uint16_t *v, long long rows, int cols,
                             uint8_t *nib, uint8_t *sc, hipStream_t s);
hipError_t launch_quant_f32(const float *v, long long rows, int cols,
                            uint8_t *nib, uint8_t *sc, hipStream_t s);
hipError_t launch_prefill_gate_up(const uint8_t *xq, const uint8_t *xsc,
                                  const uint8_t *const *experts,
                                  const PermOut &o, int max_items, int hidden,
                                  int inter, uint8_t *hq, uint8_t *hsc,
                                  float *h32, hipStream_t s);
hipError_t launch_prefill_down(const uint8_t *hq, const uint8_t *hsc,
                               const uint8_t *const *experts, const PermOut &o,
                               int max_items, int hidden, int inter, float *yp,
                               hipStream_t s);
// LDS scratch of one wave's top-k (k3_topk.h).
struct TopkLds {
  double cand_key[64];
  int cand_idx[64];
  double ranked[K3_MAX_TOPK];
};
constexpr int kFusedTopkMaxExperts = 16 * 64;  // n handled by the fused path
// LDS of the workgroup-parallel top-k (one expert per thread, n <= 1024).
struct TopkWgLds {
  uint32_t okey[kFusedTopkMaxExperts];  // keys as ordered fp32 (rounded down)
  int gt[64], ge[64], rank[64], wave_cnt[16];
  double cand_key[64];
  int cand_idx[64];
  double sel_key[K3_MAX_TOPK], ranked[K3_MAX_TOPK];
  int sel[K3_MAX_TOPK];
  float wt[K3_MAX_TOPK];
  int wt_later;  // the weights are left to topk_wg_weights
  TopkLds tk;    // the single-wave fallback
};
// The decode layer's first expert stage with top-k folded in (k3_expert.hip).
hipError_t launch_gate_up_routed(const uint16_t *x, const double *logits,
                                 const uint8_t *const *experts, int n, int k,
                                 int hidden, int inter, float *h, int32_t *idx,
                                 float *w, hipStream_t s);
// Dequantise-then-multiply control (k3_dense.hip).
hipError_t launch_dequant_expert(const uint8_t *blob, int hidden, int inter,
                                 float *dense, hipStream_t s);
hipError_t launch_experts_dense(const uint16_t *x, const float *const *table,
                                const int32_t *idx, int k, int hidden, int inter,
                                float *h, float *yp, hipStream_t s);
hipError_t launch_combine(const float *yp, const float *w, int k, int hidden,
                          uint16_t *y, float *y_f32, hipStream_t s,
                          const float *add = nullptr);
// Shared experts (k3_shared.hip): h [n_shared][inter], ys [hidden] = the sum
// of their outputs.
hipError_t launch_shared_experts(const uint16_t *x, const uint16_t *const *shared,
                                 int n_shared, int hidden, int inter, float *h,
                                 float *ys, hipStream_t s);
// One token's router logits and the shared experts' h in one launch, then
// their down stage (the two halves of launch_router + launch_shared_experts).
hipError_t launch_router_shared(const uint16_t *x, const uint16_t *R, int hidden,
                                int n_experts, double *logits,
                                const uint16_t *const *shared, int n_shared, int inter,
                                float *h, hipStream_t s);
hipError_t launch_shared_down(const float *h, const uint16_t *const *shared, int n_shared,
                              int hidden, int inter, float *ys, hipStream_t s);
// The decode layer's expert work in one launch (k3_expert.hip): top-k of
// the logits, gate/up, down, combine. slots: 2 * kMaxSyncGrid arrival words
// (moe_experts_grid() <= kMaxSyncGrid workgroups); val: this call's value,
// never reused in the process.
// Work items spread over the XCDs. Workgroups are dealt to the eight XCDs
// round-robin by index (b % 8 runs on XCD b % 8), and each XCD has its own
// L2. With a grid of xcd_grid(items, units) workgroups, xcd_unit(b, units)
// gives workgroup b the unit item * units + j of item 8 (p / units) + b % 8,
// j = p % units, p = b / 8: XCD x takes items x, x + 8, ... with all of an
// item's units, so the activations an item's workgroups share come into one
// L2 once, and every XCD gets an equal share of the items.
constexpr int kXcds = 8;
inline long long xcd_grid(long long items, long long units) {
  return kXcds * ((items + kXcds - 1) / kXcds) * units;
}
__device__ __forceinline__ int xcd_unit(int b, int units) {
  const int x = b % kXcds, p = b / kXcds;
  return (kXcds * (p / units) + x) * units + p % units;
}

constexpr int kMaxSyncGrid = 1024;
constexpr int kMaxDevices = 64;  // per-device state of the library
// Runs `launch` (which enqueues one grid whose workgroups wait for each
// other, on stream s) so that no two such grids overlap on the device
// (k3_expert.hip).
hipError_t grid_sync_launch(hipStream_t s, const std::function<hipError_t()> &launch);
unsigned moe_experts_grid();
// Poll limits of the hand-off waits on the current device: the expert
// launch (k3_expert.hip) and the one-expert launch (k3_expert_one.hip).
hipError_t set_expert_wait_limit(int polls);
hipError_t set_expert_one_wait_limit(int polls);
// The shared experts' down stage taken inside the expert launch: hs [n][inter]
// from an earlier launch, ys [hidden] written here and added by the combine.
struct SharedStage {
  const float *hs;
  const uint16_t *const *shared;
  int n_shared, inter;
  float *ys;
};
hipError_t launch_moe_experts(const uint16_t *x, const double *logits,
                              const uint8_t *const *experts, int n, int k,
                              int hidden, int inter, float *h, float *yp,
                              uint64_t *slots, uint64_t val, int32_t *idx,
                              float *w, uint16_t *y, float *y_f32,
                              hipStream_t s, const float *add = nullptr,
                              const SharedStage *sh = nullptr);
// One expert in one launch over every compute unit (k3_expert_one.hip):
// gate/up split along K into expert_one_split() chunks per tile, one
// hand-off, then down. ws: expert_one_workspace_bytes() (partials, then
// kMaxSyncGrid arrival words);
// val: a per-call value.
int expert_one_split(int hidden, int inter);
size_t expert_one_workspace_bytes(int hidden, int inter);
hipError_t launch_expert_one(const uint16_t *x, const uint8_t *expert, int hidden, int inter,
                             float *y, float *h, void *ws, uint64_t val, hipStream_t s);
// Calibration read of `bytes` (a multiple of 16) at `buf` (k3_probe.hip).
hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);
// Pinned host buffer of at least n ints owned by an expert cache
// (k3_cache.hip), grown on demand (NULL if that fails): where the cached
// layers receive a selection.
int32_t *cache_selection_buffer(k3_cache_t c, size_t n);
hipError_t launch_router(const uint16_t *x, const uint16_t *R, int T,
                         int hidden, int n, double *logits, hipStream_t s);
// scale multiplies the renormalised weights (1: none).
hipError_t launch_topk_f64(const double *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s, double scale = 1.0);
hipError_t launch_topk_f32(const float *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s);

}  // namespace k3
