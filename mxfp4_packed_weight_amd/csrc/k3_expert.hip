// MXFP4 matrix-vector kernels: plain GEMV, the routed expert's gate/up +
// SwiGLU stage, its down stage and the weighted combine.
//
// The matrix kernels are CU-persistent: the grid has one workgroup of kNW
// waves per compute unit, each workgroup owns a contiguous range of 64-row
// tiles (of one matrix, or of the k selected experts back to back) and
// streams it through run_rows (k3_stream.h), which converts the codes in
// registers and multiplies them by wave-uniform activations on the vector
// ALU. Each row's sum has one fixed order that depends on the shape and grid
// only, so reruns are bit-identical (the pages' rule that every row is summed
// by one owner in one order, [SAT] "A floating-point contract, not a
// convention"). The work is a memory-bound stream of packed bytes ("the wait
// is for bytes to arrive", [SAT] "Reduction one").
#include "k3_stream.h"
#include "k3_sync.h"
#include "k3_topk.h"

namespace k3 {

namespace {

constexpr int kThreads = kNW * 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__global__ __launch_bounds__(kThreads) void gemv_f32_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ tiles, int rows,
    int cols, float *__restrict__ y) {
  __shared__ float part[kPartFloats];
  const MatLayout m = mat_layout(rows, cols);
  int t0, t1;
  wg_range(m.ntiles, &t0, &t1);
  run_rows(
      t0, t1, m.G, m.G4,
      [&](int t) { return tiles + (size_t)t * m.tile_bytes; },
      [&](u32x4 w, int g, int) { return group_dot_f32(w, x + (size_t)32 * g); },
      [&](int t, int lane, float s) {
        const int row = t * kTileRows + lane;
        if (row < rows) y[row] = s;
      },
      part);
}

__device__ __forceinline__ const uint8_t *expert_base(
    const uint8_t *const *__restrict__ experts, const int32_t *__restrict__ idx,
    const uint8_t *single, int slot) {
  return experts ? experts[idx[slot]] : single;
}

// Tiles of the k slots back to back: tile t is gate/up tile t % T of slot
// t / T (T tiles per expert). h[j][i] = SiLU(gate_i . x) * (up_i . x).
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t *__restrict__ x, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ h) {
  __shared__ float part[kPartFloats];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.gu.ntiles;
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  run_rows(
      t0, t1, L.gu.G, L.gu.G4,
      [&](int t) {
        return expert_base(experts, idx, single, t / T) +
               (size_t)(t % T) * L.gu.tile_bytes;
      },
      [&](u32x4 w, int g, int) { return group_dot_bf16(w, xp + (size_t)16 * g); },
      [&](int t, int lane, float s) {
        const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
        int is_up, row;
        gu_lane_row(t % T, lane, &is_up, &row);
        if (lane < 32 && row < inter) h[(size_t)(t / T) * inter + row] = silu(s) * u;
      },
      part);
}

// yp[j][r] = W_down(e_j)[r] . h[j], tiles of the k slots back to back (a
// workgroup's tiles share one or two slots, so its activations stay within
// the scalar cache).
__global__ __launch_bounds__(kThreads) void down_kernel(
    const float *__restrict__ h, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ yp) {
  __shared__ float part[kPartFloats];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.down.ntiles;
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  run_rows(
      t0, t1, L.down.G, L.down.G4,
      [&](int t) {
        return expert_base(experts, idx, single, t / T) + L.down_offset +
               (size_t)(t % T) * L.down.tile_bytes;
      },
      [&](u32x4 w, int g, int t) {
        return group_dot_f32(w, h + (size_t)(t / T) * inter + (size_t)32 * g);
      },
      [&](int t, int lane, float s) {
        const int row = (t % T) * kTileRows + lane;
        if (row < hidden) yp[(size_t)(t / T) * hidden + row] = s;
      },
      part);
}

// The decode layer's first expert stage with the selection folded in:
// every workgroup ranks the token's n logits itself with all of its waves
// (topk_wg: the same selection everywhere, so no grid-wide step is needed),
// workgroup 0 publishes idx and w, then the tiles of the k selected
// experts' gate/up stacks are streamed as in gate_up_kernel. One launch
// fewer than a separate top-k.
__global__ __launch_bounds__(kThreads) void gate_up_routed_kernel(
    const uint16_t *__restrict__ x, const double *__restrict__ logits,
    const uint8_t *const *__restrict__ experts, int n, int k, int hidden,
    int inter, float *__restrict__ h, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out) {
  __shared__ float part[kPartFloats];
  __shared__ TopkWgLds tk;
  topk_wg<kNW>(logits, n, k, tk);
  if (blockIdx.x == 0 && threadIdx.x < k) {
    idx_out[threadIdx.x] = tk.sel[threadIdx.x];
    w_out[threadIdx.x] = tk.wt[threadIdx.x];
  }
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.gu.ntiles;
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
  int t0, t1;
  wg_range(k * T, &t0, &t1);
  run_rows(
      t0, t1, L.gu.G, L.gu.G4,
      [&](int t) {
        const int e = __builtin_amdgcn_readfirstlane(tk.sel[t / T]);
        return ldc(experts + e) + (size_t)(t % T) * L.gu.tile_bytes;
      },
      [&](u32x4 w, int g, int) { return group_dot_bf16(w, xp + (size_t)16 * g); },
      [&](int t, int lane, float s) {
        const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
        int is_up, row;
        gu_lane_row(t % T, lane, &is_up, &row);
        if (lane < 32 && row < inter) h[(size_t)(t / T) * inter + row] = silu(s) * u;
      },
      part);
}

// The decode layer's last stage: down projection and weighted combine in
// one launch. The down tiles are those of down_kernel on the same grid;
// their partials go out with device-coherent stores, and each workgroup
// then marks its arrival slot with the call's value `val`. Row tile r's
// partials are tiles s * T + r (s < k); the workgroup that owns the last
// one (slot k - 1) waits for the owners of the others and sums them in rank
// order exactly as combine_kernel, so the bits equal down_kernel followed by
// combine_kernel. Every workgroup waited for has a lower index and waits
// for nothing itself, so the waits end even if the grid is not all resident
// at once; a wait that still runs out (~1 s) makes the call write NaN.
__global__ __launch_bounds__(kThreads) void down_combine_kernel(
    const float *__restrict__ h, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const float *__restrict__ w, int k,
    int hidden, int inter, float *yp, uint64_t *slots, uint64_t val,
    uint16_t *__restrict__ y, float *__restrict__ y_f32) {
  __shared__ float part[kPartFloats];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.down.ntiles, total = k * T;
  int t0, t1;
  wg_range(total, &t0, &t1);
  run_rows(
      t0, t1, L.down.G, L.down.G4,
      [&](int t) {
        return ldc(experts + ldc(idx + t / T)) + L.down_offset +
               (size_t)(t % T) * L.down.tile_bytes;
      },
      [&](u32x4 wv, int g, int t) {
        return group_dot_f32(wv, h + (size_t)(t / T) * inter + (size_t)32 * g);
      },
      [&](int t, int lane, float s) {
        const int row = (t % T) * kTileRows + lane;
        if (row < hidden) st_dev(yp + (size_t)(t / T) * hidden + row, s);
      },
      part);
  arrive(slots, val);
  const int lane = threadIdx.x & 63;
  const int last = (k - 1) * T;
  const int r_lo = max(t0 - last, 0), r_hi = min(t1 - last, T);
  for (int r = r_lo + wave_id(); r < r_hi; r += kNW) {
    const int owner = lane < k ? tile_owner(lane * T + r, total, gridDim.x) : 0;
    if (!wave_wait_owners(slots, owner, k, val) && lane == 0) bad = 1;
    const int row = r * kTileRows + lane;
    if (row < hidden) {
      float acc = 0.f;
      for (int j0 = 0; j0 < k; j0 += 16) {  // as combine_kernel
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          v[j] = j0 + j < k ? ld_dev(yp + (size_t)(j0 + j) * hidden + row) : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j0 + j < k) acc = fmaf(w[j0 + j], v[j], acc);
      }
      if (y_f32) y_f32[row] = acc;
      if (y) y[row] = f32_to_bf16_rne(acc);
    }
  }
  __syncthreads();
  if (bad)  // the outputs cannot be trusted: say so in them
    for (int i = threadIdx.x; i < hidden; i += kThreads) {
      if (y_f32) y_f32[i] = __builtin_nanf("");
      if (y) y[i] = 0x7FC0;
    }
}

// y[i] = sum_j w[j] * yp[j][i] in rank order j = 0..k-1, then bf16 (RNE).
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ yp, const float *__restrict__ w, int k,
    int hidden, uint16_t *__restrict__ y, float *__restrict__ y_f32) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= hidden) return;
  float acc = 0.f;
  for (int j0 = 0; j0 < k; j0 += 16) {  // issue a batch of loads, then add
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = j0 + j < k ? yp[(size_t)(j0 + j) * hidden + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j0 + j < k) acc = fmaf(w[j0 + j], v[j], acc);
  }
  if (y_f32) y_f32[i] = acc;
  if (y) y[i] = f32_to_bf16_rne(acc);
}

#ifndef K3_WG_PER_CU
#define K3_WG_PER_CU 1
#endif
unsigned grid_for_tiles(int total) {
  const int wgs = num_cus() * K3_WG_PER_CU;
  return (unsigned)(total < wgs ? total : wgs);
}

}  // namespace

hipError_t launch_gemv_f32(const float *x, const uint8_t *tiles, int rows,
                           int cols, float *y, hipStream_t s) {
  const MatLayout m = mat_layout(rows, cols);
  hipLaunchKernelGGL(gemv_f32_kernel, dim3(grid_for_tiles(m.ntiles)),
                     dim3(kThreads), 0, s, x, tiles, rows, cols, y);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t *x, const uint8_t *const *experts,
                          const int32_t *idx, const uint8_t *single,
                          int nslots, int hidden, int inter, float *h,
                          hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(gate_up_kernel,
                     dim3(grid_for_tiles(nslots * L.gu.ntiles)), dim3(kThreads),
                     0, s, x, experts, idx, single, nslots, hidden, inter, h);
  return hipGetLastError();
}

hipError_t launch_down(const float *h, const uint8_t *const *experts,
                       const int32_t *idx, const uint8_t *single, int nslots,
                       int hidden, int inter, float *yp, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(down_kernel,
                     dim3(grid_for_tiles(nslots * L.down.ntiles)),
                     dim3(kThreads), 0, s, h, experts, idx, single, nslots,
                     hidden, inter, yp);
  return hipGetLastError();
}

hipError_t launch_gate_up_routed(const uint16_t *x, const double *logits,
                                 const uint8_t *const *experts, int n, int k,
                                 int hidden, int inter, float *h, int32_t *idx,
                                 float *w, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(gate_up_routed_kernel, dim3(grid_for_tiles(k * L.gu.ntiles)),
                     dim3(kThreads), 0, s, x, logits, experts, n, k, hidden,
                     inter, h, idx, w);
  return hipGetLastError();
}

hipError_t launch_down_combine(const float *h, const uint8_t *const *experts,
                               const int32_t *idx, const float *w, int k,
                               int hidden, int inter, float *yp,
                               uint64_t *slots, uint64_t val, uint16_t *y,
                               float *y_f32, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(down_combine_kernel,
                     dim3(grid_for_tiles(k * L.down.ntiles)), dim3(kThreads),
                     0, s, h, experts, idx, w, k, hidden, inter, yp, slots, val,
                     y, y_f32);
  return hipGetLastError();
}

unsigned down_combine_grid(int k, int hidden, int inter) {
  return grid_for_tiles(k * expert_layout(hidden, inter).down.ntiles);
}

hipError_t launch_combine(const float *yp, const float *w, int k, int hidden,
                          uint16_t *y, float *y_f32, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3((hidden + 255) / 256), dim3(256), 0,
                     s, yp, w, k, hidden, y, y_f32);
  return hipGetLastError();
}

}  // namespace k3
