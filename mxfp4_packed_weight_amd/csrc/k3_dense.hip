// Control path: the routed expert multiplied from dequantised fp32 copies.
//
// The pages' engine never expands an expert: one expert is 17.55 MB packed
// and would be 132 MB as floats, 7.5 times the bytes, and since the product
// waits on bytes, about 7.5 times the time ([SAT] "Reduction one"; [SAT] "The
// cache the project exists for"). These kernels exist to measure that gap on
// this part: k3_expert_dequantize writes an expert's three matrices as dense
// row-major fp32, and k3_experts_dense runs the same SwiGLU experts from such
// copies. They are not on the packed path.
//
// Dense blob of one expert: gate [inter][hidden], up [inter][hidden], down
// [hidden][inter], fp32, back to back. A weight is E2M1(code) * 2^(e-127)
// (exact in fp32 for exponent bytes 0..252); a group whose exponent byte is
// 255 is written as zeros (it contributes nothing to a product).
#include "k3_decode.h"
#include "k3_internal.h"

namespace k3 {

namespace {

typedef float f32v4 __attribute__((ext_vector_type(4)));

// One wave per (64-row tile, group): lane r converts its row's 32 codes and
// writes them as 128 contiguous bytes. Loads are the tile's contiguous KiB.
// rowmap(t, lane, &dst_row_ptr_or_null) names where a lane's row goes.
template <class RowMap>
__device__ __forceinline__ void dequant_group(const uint8_t *tiles, const MatLayout &m,
                                              int t, int g, RowMap rowmap) {
  const int lane = threadIdx.x & 63;
  float *dst = rowmap(t, lane);
  if (!dst) return;
  const uint8_t *tb = tiles + (size_t)t * m.tile_bytes;
  const u32x4 w = *(const u32x4 *)(tb + code_offset(g, lane));
  const uint32_t e = tb[scale_offset(g, lane)];
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float4 *o = reinterpret_cast<float4 *>(dst + (size_t)32 * g);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 3);
    const int s = (int)e - 127;
    float4 a, b;
    a.x = ldexpf(v0.x, s);
    a.y = ldexpf(v0.y, s);
    a.z = ldexpf(v1.x, s);
    a.w = ldexpf(v1.y, s);
    b.x = ldexpf(v2.x, s);
    b.y = ldexpf(v2.y, s);
    b.z = ldexpf(v3.x, s);
    b.w = ldexpf(v3.y, s);
    if (e == 255u) a = b = make_float4(0.f, 0.f, 0.f, 0.f);
    o[2 * d] = a;
    o[2 * d + 1] = b;
  }
}

// Blocks of one wave; block b is (tile b / G, group b % G) of the gate/up
// stack, then of the down matrix.
__global__ __launch_bounds__(64) void dequant_expert_kernel(const uint8_t *__restrict__ blob,
                                                            int hidden, int inter,
                                                            float *__restrict__ dense) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const int ngu = L.gu.ntiles * L.gu.G;
  int b = blockIdx.x;
  if (b < ngu) {
    float *gate = dense, *up = dense + (size_t)inter * hidden;
    dequant_group(blob, L.gu, b / L.gu.G, b % L.gu.G, [&](int t, int lane) -> float * {
      int is_up, row;
      gu_lane_row(t, lane, &is_up, &row);
      if (row >= inter) return nullptr;
      return (is_up ? up : gate) + (size_t)row * hidden;
    });
    return;
  }
  b -= ngu;
  float *down = dense + (size_t)2 * inter * hidden;
  dequant_group(blob + L.down_offset, L.down, b / L.down.G, b % L.down.G,
                [&](int t, int lane) -> float * {
                  const int row = t * kTileRows + lane;
                  return row < hidden ? down + (size_t)row * inter : nullptr;
                });
}

// Sum over the 64 lanes in a fixed butterfly order (the same on every run).
__device__ __forceinline__ float wave_sum_fixed(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr int kDenseWaves = 4;

// One wave per (slot j, h row i): lane l accumulates columns 4l + 256m
// (m ascending) of the gate and up rows, the lanes are summed in a fixed
// order, h = SiLU(g) * u.
__global__ __launch_bounds__(64 * kDenseWaves) void dense_gate_up_kernel(
    const uint16_t *__restrict__ x, const float *const *__restrict__ table,
    const int32_t *__restrict__ idx, int k, int hidden, int inter,
    float *__restrict__ h) {
  const int gw = blockIdx.x * kDenseWaves + (threadIdx.x >> 6);
  if (gw >= k * inter) return;
  const int lane = threadIdx.x & 63, j = gw / inter, i = gw % inter;
  const float *blob = table[idx[j]];
  const f32v4 *gr = reinterpret_cast<const f32v4 *>(blob + (size_t)i * hidden);
  const f32v4 *ur = reinterpret_cast<const f32v4 *>(blob + (size_t)(inter + i) * hidden);
  const uint2 *xv = reinterpret_cast<const uint2 *>(x);
  float ag = 0.f, au = 0.f;
#pragma unroll 4
  for (int c4 = lane; 4 * c4 < hidden; c4 += 64) {
    const f32v4 g = __builtin_nontemporal_load(gr + c4);
    const f32v4 u = __builtin_nontemporal_load(ur + c4);
    const uint2 xb = xv[c4];
    const float x0 = __uint_as_float(xb.x << 16), x1 = __uint_as_float(xb.x & 0xFFFF0000u);
    const float x2 = __uint_as_float(xb.y << 16), x3 = __uint_as_float(xb.y & 0xFFFF0000u);
    ag = fmaf(g.x, x0, ag);
    ag = fmaf(g.y, x1, ag);
    ag = fmaf(g.z, x2, ag);
    ag = fmaf(g.w, x3, ag);
    au = fmaf(u.x, x0, au);
    au = fmaf(u.y, x1, au);
    au = fmaf(u.z, x2, au);
    au = fmaf(u.w, x3, au);
  }
  ag = wave_sum_fixed(ag);
  au = wave_sum_fixed(au);
  if (lane == 0) h[(size_t)j * inter + i] = silu(ag) * au;
}

// One wave per (slot j, output row r) of the down matrices.
__global__ __launch_bounds__(64 * kDenseWaves) void dense_down_kernel(
    const float *__restrict__ h, const float *const *__restrict__ table,
    const int32_t *__restrict__ idx, int k, int hidden, int inter,
    float *__restrict__ yp) {
  const int gw = blockIdx.x * kDenseWaves + (threadIdx.x >> 6);
  if (gw >= k * hidden) return;
  const int lane = threadIdx.x & 63, j = gw / hidden, r = gw % hidden;
  const float *blob = table[idx[j]];
  const f32v4 *dr =
      reinterpret_cast<const f32v4 *>(blob + (size_t)2 * inter * hidden + (size_t)r * inter);
  const f32v4 *hv = reinterpret_cast<const f32v4 *>(h + (size_t)j * inter);
  float a = 0.f;
#pragma unroll 2
  for (int c4 = lane; 4 * c4 < inter; c4 += 64) {
    const f32v4 w = __builtin_nontemporal_load(dr + c4);
    const f32v4 v = hv[c4];
    a = fmaf(w.x, v.x, a);
    a = fmaf(w.y, v.y, a);
    a = fmaf(w.z, v.z, a);
    a = fmaf(w.w, v.w, a);
  }
  a = wave_sum_fixed(a);
  if (lane == 0) yp[(size_t)j * hidden + r] = a;
}

}  // namespace

hipError_t launch_dequant_expert(const uint8_t *blob, int hidden, int inter,
                                 float *dense, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const unsigned blocks = (unsigned)(L.gu.ntiles * L.gu.G + L.down.ntiles * L.down.G);
  hipLaunchKernelGGL(dequant_expert_kernel, dim3(blocks), dim3(64), 0, s, blob, hidden,
                     inter, dense);
  return hipGetLastError();
}

hipError_t launch_experts_dense(const uint16_t *x, const float *const *table,
                                const int32_t *idx, int k, int hidden, int inter,
                                float *h, float *yp, hipStream_t s) {
  const unsigned b1 = (unsigned)(((size_t)k * inter + kDenseWaves - 1) / kDenseWaves);
  hipLaunchKernelGGL(dense_gate_up_kernel, dim3(b1), dim3(64 * kDenseWaves), 0, s, x, table,
                     idx, k, hidden, inter, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned b2 = (unsigned)(((size_t)k * hidden + kDenseWaves - 1) / kDenseWaves);
  hipLaunchKernelGGL(dense_down_kernel, dim3(b2), dim3(64 * kDenseWaves), 0, s, h, table, idx,
                     k, hidden, inter, yp);
  return hipGetLastError();
}

}  // namespace k3
