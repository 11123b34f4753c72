// MXFP4 matrix-vector kernels: plain GEMV, the routed expert's gate/up +
// SwiGLU stage, its down stage, and the weighted combine.
//
// The matrix kernels are CU-persistent: the grid has one workgroup of kNW
// waves per compute unit, each workgroup owns a contiguous range of 64-row
// tiles (of one matrix, or of the k selected experts back to back) and
// streams it with run_tiles (k3_decode.h). Each row's sum has one fixed order
// that depends on the shape only, so reruns are bit-identical (the pages'
// rule that every row is summed by one owner in one order, [SAT] "A
// floating-point contract, not a convention"). The work is a memory-bound
// stream of packed bytes ("the wait is for bytes to arrive", [SAT]
// "Reduction one").
#include "k3_decode.h"
#include "k3_internal.h"

namespace k3 {

namespace {

constexpr int kThreads = kNW * 64;
#ifndef K3_ACT_LDS
#define K3_ACT_LDS 0
#endif

// Copies n 32-bit words from global memory to LDS with the whole workgroup.
__device__ __forceinline__ void stage_words(uint32_t *dst, const uint32_t *src,
                                            int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void gemv_f32_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ tiles, int rows,
    int cols, float *__restrict__ y) {
  const MatLayout m = mat_layout(rows, cols);
  int t0, t1;
  wg_range(m.ntiles, &t0, &t1);
  run_tiles(
      t0, t1, m.G, m.G4,
      [&](int t) { return tiles + (size_t)t * m.tile_bytes; },
      [&](u32x4 w, int g, int) { return group_dot_f32(w, x + (size_t)32 * g); },
      [&](int t, int lane, float s) {
        const int row = t * kTileRows + lane;
        if (row < rows) y[row] = s;
      });
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

__device__ __forceinline__ const uint8_t *expert_base(
    const uint8_t *const *__restrict__ experts, const int32_t *__restrict__ idx,
    const uint8_t *single, int slot) {
  return experts ? experts[idx[slot]] : single;
}

// Tiles of the k slots back to back: tile t is gate/up tile t % T of slot
// t / T (T tiles per expert). h[j][i] = SiLU(gate_i . x) * (up_i . x).
// x is staged once per workgroup in LDS (hidden/2 words, dynamic LDS).
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t *__restrict__ x, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ h) {
  extern __shared__ uint32_t act[];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.gu.ntiles;
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
#if K3_ACT_LDS
  stage_words(act, xp, hidden / 2);
  __syncthreads();
#endif
  run_tiles(
      t0, t1, L.gu.G, L.gu.G4,
      [&](int t) {
        return expert_base(experts, idx, single, t / T) +
               (size_t)(t % T) * L.gu.tile_bytes;
      },
      [&](u32x4 w, int g, int) {
#if K3_ACT_LDS
        return group_dot_bf16_lds(w, act + (size_t)16 * g);
#else
        return group_dot_bf16(w, xp + (size_t)16 * g);
#endif
      },
      [&](int t, int lane, float s) {
        const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
        int is_up, row;
        gu_lane_row(t % T, lane, &is_up, &row);
        if (lane < 32 && row < inter)
          h[(size_t)(t / T) * inter + row] = silu(s) * u;
      });
}

// yp[j][r] = W_down(e_j)[r] . h[j], tiles of the k slots back to back. The
// workgroup's range is walked slot by slot with h[j] staged in LDS
// (inter words, dynamic LDS).
__global__ __launch_bounds__(kThreads) void down_kernel(
    const float *__restrict__ h, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ yp) {
  extern __shared__ uint32_t act[];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.down.ntiles;
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  const float *hs = reinterpret_cast<const float *>(act);
  for (int a = t0; a < t1;) {
    const int j = a / T;
    const int b = min(t1, (j + 1) * T);
#if K3_ACT_LDS
    __syncthreads();
    stage_words(act, reinterpret_cast<const uint32_t *>(h + (size_t)j * inter),
                inter);
    __syncthreads();
#endif
    run_tiles(
        a, b, L.down.G, L.down.G4,
        [&](int t) {
          return expert_base(experts, idx, single, j) + L.down_offset +
                 (size_t)(t % T) * L.down.tile_bytes;
        },
        [&](u32x4 w, int g, int) {
#if K3_ACT_LDS
          return group_dot_f32_lds(w, hs + (size_t)32 * g);
#else
          return group_dot_f32(w, h + (size_t)j * inter + (size_t)32 * g);
#endif
        },
        [&](int t, int lane, float s) {
          const int row = (t % T) * kTileRows + lane;
          if (row < hidden) yp[(size_t)j * hidden + row] = s;
        });
    a = b;
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

unsigned grid_for_tiles(int total) {
  const int cus = num_cus();
  return (unsigned)(total < cus ? total : cus);
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
                     K3_ACT_LDS ? (size_t)hidden * 2 : 0, s, x, experts, idx,
                     single, nslots, hidden, inter, h);
  return hipGetLastError();
}

hipError_t launch_down(const float *h, const uint8_t *const *experts,
                       const int32_t *idx, const uint8_t *single, int nslots,
                       int hidden, int inter, float *yp, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(down_kernel,
                     dim3(grid_for_tiles(nslots * L.down.ntiles)),
                     dim3(kThreads), K3_ACT_LDS ? (size_t)inter * 4 : 0, s, h,
                     experts, idx, single, nslots, hidden, inter, yp);
  return hipGetLastError();
}

hipError_t launch_combine(const float *yp, const float *w, int k, int hidden,
                          uint16_t *y, float *y_f32, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3((hidden + 255) / 256), dim3(256), 0,
                     s, yp, w, k, hidden, y, y_f32);
  return hipGetLastError();
}

}  // namespace k3
