// MXFP4 matrix-vector kernels: plain GEMV, the routed expert's gate/up +
// SwiGLU stage, its down stage, the activation-fragment builder and the
// weighted combine.
//
// The matrix kernels are CU-persistent: the grid has one workgroup of kNW
// waves per compute unit, each workgroup owns a contiguous range of 64-row
// tiles (of one matrix, or of the k selected experts back to back) and
// streams it through the FP4 matrix unit (run_tiles_mfma, k3_mfma.h). Each
// row's sum has one fixed order that depends on the shape only, so reruns
// are bit-identical (the pages' rule that every row is summed by one owner
// in one order, [SAT] "A floating-point contract, not a convention"). The
// work is a memory-bound stream of packed bytes ("the wait is for bytes to
// arrive", [SAT] "Reduction one").
#include "k3_mfma.h"

namespace k3 {

namespace {

constexpr int kThreads = kNW * 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Any flag set among n ints (wave-uniform).
__device__ __forceinline__ bool any_flag(const int *__restrict__ flags, int n) {
  int f = 0;
  for (int i = 0; i < n; ++i) f |= flags[i];
  return f != 0;
}

// This lane's B fragment of K block q from a compact fragment array.
template <int P>
__device__ __forceinline__ void load_frag(const uint8_t *frag, int q,
                                          u32x4 &b0, u32x4 &b1, uint32_t &bsc) {
  const int lane = threadIdx.x & 63, c = lane & 15, h = lane >> 4;
  const uint8_t *f = frag + (size_t)frag_bytes(P) * q;
  if (c < P) {
    const u32x4 *s = reinterpret_cast<const u32x4 *>(f + 32 * (h * P + c));
    b0 = s[0];
    b1 = s[1];
    bsc = f[128 * P + h * P + c];
  } else {
    b0 = u32x4{0u, 0u, 0u, 0u};
    b1 = b0;
    bsc = 127u;
  }
}

// Fragments of an activation vector: one wave per 128-element block.
template <int P, typename T>
__global__ __launch_bounds__(256) void act_frag_kernel(const T *__restrict__ v,
                                                       int len,
                                                       uint8_t *__restrict__ frag,
                                                       int *__restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int kb = blockIdx.x * 4 + wave_id();
  const int nkb = (len + 127) / 128;
  if (kb >= nkb) return;
  auto at = [&](int k) -> float {
    if (k >= len) return 0.f;
    if constexpr (sizeof(T) == 2) return bf16_to_f32(v[k]);
    else return (float)v[k];
  };
  const bool bad = make_frag<P>(at(128 * kb + lane), at(128 * kb + 64 + lane),
                                frag + (size_t)frag_bytes(P) * kb, lane);
  if (lane == 0) flags[kb] = bad ? 1 : 0;
}

__global__ __launch_bounds__(kThreads) void gemv_f32_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ tiles, int rows,
    int cols, const uint8_t *__restrict__ xfrag, const int *__restrict__ flags,
    float *__restrict__ y) {
  __shared__ float part[kPartFloats];
  const MatLayout m = mat_layout(rows, cols);
  int t0, t1;
  wg_range(m.ntiles, &t0, &t1);
  auto base = [&](int t) { return tiles + (size_t)t * m.tile_bytes; };
  auto epi = [&](int t, int lane, float s) {
    const int row = t * kTileRows + lane;
    if (row < rows) y[row] = s;
  };
  if (any_flag(flags, m.G4)) {
    run_tiles_valu(
        t0, t1, m.G, m.G4, base,
        [&](u32x4 w, int g, int) { return group_dot_f32(w, x + (size_t)32 * g); },
        epi, part);
  } else {
    run_tiles_mfma(
        t0, t1, m.G4, base,
        [&](int, int q, u32x4 &b0, u32x4 &b1, uint32_t &bsc) {
          load_frag<kPieces>(xfrag, q, b0, b1, bsc);
        },
        epi, part);
  }
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

__device__ __forceinline__ const uint8_t *expert_base(
    const uint8_t *const *__restrict__ experts, const int32_t *__restrict__ idx,
    const uint8_t *single, int slot) {
  return experts ? experts[idx[slot]] : single;
}

// Tiles of the k slots back to back: tile t is gate/up tile t % T of slot
// t / T (T tiles per expert). h[j][i] = SiLU(gate_i . x) * (up_i . x).
// xfrag/flags: fragments of x (act_frag_kernel).
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t *__restrict__ x, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, const uint8_t *__restrict__ xfrag,
    const int *__restrict__ flags, float *__restrict__ h) {
  __shared__ float part[kPartFloats];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.gu.ntiles;
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  auto base = [&](int t) {
    return expert_base(experts, idx, single, t / T) +
           (size_t)(t % T) * L.gu.tile_bytes;
  };
  auto epi = [&](int t, int lane, float s) {
    const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
    int is_up, row;
    gu_lane_row(t % T, lane, &is_up, &row);
    if (lane < 32 && row < inter) h[(size_t)(t / T) * inter + row] = silu(s) * u;
  };
  if (any_flag(flags, L.gu.G4)) {
    const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
    run_tiles_valu(
        t0, t1, L.gu.G, L.gu.G4, base,
        [&](u32x4 w, int g, int) { return group_dot_bf16(w, xp + (size_t)16 * g); },
        epi, part);
  } else {
    run_tiles_mfma(
        t0, t1, L.gu.G4, base,
        [&](int, int q, u32x4 &b0, u32x4 &b1, uint32_t &bsc) {
          load_frag<kPieces>(xfrag, q, b0, b1, bsc);
        },
        epi, part);
  }
}

// yp[j][r] = W_down(e_j)[r] . h[j], tiles of the k slots back to back. The
// workgroup's range is walked slot by slot; for each slot the workgroup
// first builds the 6-piece fragments of h[j] in LDS (dynamic LDS of
// ceil(inter/128) fragments).
__global__ __launch_bounds__(kThreads) void down_kernel(
    const float *__restrict__ h, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ yp) {
  extern __shared__ uint8_t hfrag[];
  __shared__ float part[kPartFloats];
  __shared__ int hbad;
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.down.ntiles;
  const int nkb = L.down.G4;
  const int lane = threadIdx.x & 63, wave = wave_id();
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  for (int a = t0; a < t1;) {
    const int j = a / T;
    const int b = min(t1, (j + 1) * T);
    const float *hj = h + (size_t)j * inter;
    __syncthreads();
    if (threadIdx.x == 0) hbad = 0;
    __syncthreads();
    for (int kb = wave; kb < nkb; kb += kNW) {
      const int k0 = 128 * kb + lane, k1 = k0 + 64;
      const bool bad = make_frag<kPieces>(
          k0 < inter ? hj[k0] : 0.f, k1 < inter ? hj[k1] : 0.f,
          hfrag + (size_t)frag_bytes(kPieces) * kb, lane);
      if (bad && lane == 0) hbad = 1;
    }
    __syncthreads();
    auto base = [&](int t) {
      return expert_base(experts, idx, single, j) + L.down_offset +
             (size_t)(t % T) * L.down.tile_bytes;
    };
    auto epi = [&](int t, int ln, float s) {
      const int row = (t % T) * kTileRows + ln;
      if (row < hidden) yp[(size_t)j * hidden + row] = s;
    };
    if (hbad) {
      run_tiles_valu(
          a, b, L.down.G, L.down.G4, base,
          [&](u32x4 w, int g, int) { return group_dot_f32(w, hj + (size_t)32 * g); },
          epi, part);
    } else {
      run_tiles_mfma(
          a, b, L.down.G4, base,
          [&](int, int q, u32x4 &b0, u32x4 &b1, uint32_t &bsc) {
            load_frag<kPieces>(hfrag, q, b0, b1, bsc);
          },
          epi, part);
    }
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

size_t act_frag_bytes(int len, int pieces) {
  return (size_t)((len + 127) / 128) * frag_bytes(pieces);
}

hipError_t launch_act_frag_bf16(const uint16_t *v, int len, uint8_t *frag,
                                int *flags, hipStream_t s) {
  const int nkb = (len + 127) / 128;
  hipLaunchKernelGGL((act_frag_kernel<kPieces, uint16_t>),
                     dim3((nkb + 3) / 4), dim3(256), 0, s, v, len, frag, flags);
  return hipGetLastError();
}

hipError_t launch_act_frag_f32(const float *v, int len, uint8_t *frag,
                               int *flags, hipStream_t s) {
  const int nkb = (len + 127) / 128;
  hipLaunchKernelGGL((act_frag_kernel<kPieces, float>), dim3((nkb + 3) / 4),
                     dim3(256), 0, s, v, len, frag, flags);
  return hipGetLastError();
}

hipError_t launch_gemv_f32(const float *x, const uint8_t *tiles, int rows,
                           int cols, const uint8_t *xfrag, const int *flags,
                           float *y, hipStream_t s) {
  const MatLayout m = mat_layout(rows, cols);
  hipLaunchKernelGGL(gemv_f32_kernel, dim3(grid_for_tiles(m.ntiles)),
                     dim3(kThreads), 0, s, x, tiles, rows, cols, xfrag, flags,
                     y);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t *x, const uint8_t *const *experts,
                          const int32_t *idx, const uint8_t *single,
                          int nslots, int hidden, int inter,
                          const uint8_t *xfrag, const int *flags, float *h,
                          hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(gate_up_kernel,
                     dim3(grid_for_tiles(nslots * L.gu.ntiles)), dim3(kThreads),
                     0, s, x, experts, idx, single, nslots, hidden, inter,
                     xfrag, flags, h);
  return hipGetLastError();
}

hipError_t launch_down(const float *h, const uint8_t *const *experts,
                       const int32_t *idx, const uint8_t *single, int nslots,
                       int hidden, int inter, float *yp, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(down_kernel,
                     dim3(grid_for_tiles(nslots * L.down.ntiles)),
                     dim3(kThreads), act_frag_bytes(inter, kPieces), s, h,
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
