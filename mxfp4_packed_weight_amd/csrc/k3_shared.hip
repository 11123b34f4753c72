// Shared experts: SwiGLU FFNs with bf16 weights that run on every token
// beside the routed ones and stay resident ([ZOR] "How does a
// 2.78-trillion-parameter model fit in 8 GB?": two per layer, classed with
// the always-on bf16 set). Their output is added to the routed mix.
//
// Blob of one shared expert: gate [inter][hidden], up [inter][hidden], down
// [hidden][inter], bf16 row-major, back to back. The work is a plain
// HBM-bound GEMV: one wave per output row, 16-byte loads (8 weights) per
// lane, products on the dot2 bf16 path, lanes summed in a fixed order, so
// reruns are bit-identical.
#include "k3_decode.h"
#include "k3_internal.h"
#include "k3_router.h"
#include "k3_shared_row.h"

namespace k3 {

namespace {

constexpr int kSharedWaves = 4;

// 8 bf16 weights (one 16-byte load) times 8 bf16 activations, added to acc
// as four dot2 steps in order.
__device__ __forceinline__ float dot8_bf16(const uint4 w, const uint4 a, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x),
                                        __builtin_bit_cast(bf16x2, a.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y),
                                        __builtin_bit_cast(bf16x2, a.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z),
                                        __builtin_bit_cast(bf16x2, a.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w),
                                        __builtin_bit_cast(bf16x2, a.w), acc, false);
  return acc;
}

// Row gw = (shared expert s, h row i) of the gate/up stage, by one wave:
// lane l takes columns 8l + 512m (m ascending) of the gate and up rows,
// h[s][i] = SiLU(g) * u.
__device__ __forceinline__ void shared_gate_up_row(const uint16_t *__restrict__ x,
                                                   const uint16_t *const *__restrict__ shared,
                                                   int hidden, int inter, int gw,
                                                   float *__restrict__ h) {
  const int lane = threadIdx.x & 63, s = gw / inter, i = gw % inter;
  const uint16_t *blob = shared[s];
  const uint16_t *gr = blob + (size_t)i * hidden;
  const uint16_t *ur = blob + (size_t)(inter + i) * hidden;
  const uint4 *xv = reinterpret_cast<const uint4 *>(x);
  float ag = 0.f, au = 0.f;
#pragma unroll 4
  for (int c8 = lane; 8 * c8 < hidden; c8 += 64) {
    const uint4 g = ld16_nt(gr + 8 * c8), u = ld16_nt(ur + 8 * c8), a = xv[c8];
    ag = dot8_bf16(g, a, ag);
    au = dot8_bf16(u, a, au);
  }
  ag = lanes_sum(ag);
  au = lanes_sum(au);
  if (lane == 0) h[(size_t)s * inter + i] = silu(ag) * au;
}

__global__ __launch_bounds__(64 * kSharedWaves) void shared_gate_up_kernel(
    const uint16_t *__restrict__ x, const uint16_t *const *__restrict__ shared,
    int n_shared, int hidden, int inter, float *__restrict__ h) {
  const int gw = blockIdx.x * kSharedWaves + (threadIdx.x >> 6);
  if (gw < n_shared * inter) shared_gate_up_row(x, shared, hidden, inter, gw, h);
}

// The decode layer's router and the shared experts' gate/up stage in one
// launch (both are row dot products against the same token): blocks
// [0, n) are router rows (as router_kernel, the same bits), the rest take
// kSharedWaves shared rows each (as shared_gate_up_kernel). The router rows
// are dispatched first; their short latency-bound work then hides under the
// shared rows' stream instead of paying a launch of its own.
static_assert(kSharedWaves == kRouterSplit, "one block shape serves both row kinds");
__global__ __launch_bounds__(64 * kSharedWaves) void router_shared_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ R, int n_experts,
    double *__restrict__ logits, const uint16_t *const *__restrict__ shared,
    int n_shared, int hidden, int inter, float *__restrict__ h) {
  __shared__ double partial[kRouterSplit];
  if ((int)blockIdx.x < n_experts) {
    router_row_logit<true>(R + (size_t)blockIdx.x * hidden, x, hidden, partial,
                           logits + blockIdx.x);
    return;
  }
  const int gw = ((int)blockIdx.x - n_experts) * kSharedWaves + (threadIdx.x >> 6);
  if (gw < n_shared * inter) shared_gate_up_row(x, shared, hidden, inter, gw, h);
}

// One wave per output row r: ys[r] = sum over s of W_down(s)[r] . h[s]
// (shared_down_row, k3_shared_row.h).
__global__ __launch_bounds__(64 * kSharedWaves) void shared_down_kernel(
    const float *__restrict__ h, const uint16_t *const *__restrict__ shared,
    int n_shared, int hidden, int inter, float *__restrict__ ys) {
  const int r = blockIdx.x * kSharedWaves + (threadIdx.x >> 6);
  if (r >= hidden) return;
  const float acc = shared_down_row(h, shared, n_shared, hidden, inter, r);
  if ((threadIdx.x & 63) == 0) ys[r] = acc;
}

}  // namespace

hipError_t launch_router_shared(const uint16_t *x, const uint16_t *R, int hidden,
                                int n_experts, double *logits,
                                const uint16_t *const *shared, int n_shared, int inter,
                                float *h, hipStream_t s) {
  const unsigned blocks = (unsigned)(n_experts + ((size_t)n_shared * inter + kSharedWaves - 1) /
                                                     kSharedWaves);
  hipLaunchKernelGGL(router_shared_kernel, dim3(blocks), dim3(64 * kSharedWaves), 0, s, x, R,
                     n_experts, logits, shared, n_shared, hidden, inter, h);
  return hipGetLastError();
}

hipError_t launch_shared_down(const float *h, const uint16_t *const *shared, int n_shared,
                              int hidden, int inter, float *ys, hipStream_t s) {
  const unsigned b2 = (unsigned)((hidden + kSharedWaves - 1) / kSharedWaves);
  hipLaunchKernelGGL(shared_down_kernel, dim3(b2), dim3(64 * kSharedWaves), 0, s, h, shared,
                     n_shared, hidden, inter, ys);
  return hipGetLastError();
}

hipError_t launch_shared_experts(const uint16_t *x, const uint16_t *const *shared,
                                 int n_shared, int hidden, int inter, float *h,
                                 float *ys, hipStream_t s) {
  const unsigned b1 = (unsigned)(((size_t)n_shared * inter + kSharedWaves - 1) / kSharedWaves);
  hipLaunchKernelGGL(shared_gate_up_kernel, dim3(b1), dim3(64 * kSharedWaves), 0, s, x, shared,
                     n_shared, hidden, inter, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned b2 = (unsigned)((hidden + kSharedWaves - 1) / kSharedWaves);
  hipLaunchKernelGGL(shared_down_kernel, dim3(b2), dim3(64 * kSharedWaves), 0, s, h, shared,
                     n_shared, hidden, inter, ys);
  return hipGetLastError();
}

}  // namespace k3
