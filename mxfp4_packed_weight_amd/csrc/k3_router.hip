// Router: bf16 logits GEMV in fp64 and sigmoid top-k selection.
//
// Logits: one wave per (token, expert) row. Each lane issues the loads of
// all its 16-byte chunks of the bf16 router row (and of x) before computing,
// so the whole router matrix is in flight at once; products are formed in
// fp64 (a product of two bf16 values is exact there) into four chains per
// lane, and the lane sums are combined by a fixed DPP tree, so the logits
// are reproducible bit for
// bit and within ~1e-16 of a sequential fp64 sum, which keeps the top-k
// indices identical to an fp64 reference.
//
// Selection: one wave per token with the keys in registers; a cheap lower
// bound keeps ~18 candidates, which are ranked in parallel (topk_wave,
// k3_topk.h). Ties go to the lower expert index. The routing bias only
// changes the keys; the weights always come from the unbiased sigmoid scores
// ([ZOR] "How is the C engine actually built?", invariant 3), renormalised to
// sum to one, summed in rank order.
#include <limits.h>
#include <math.h>

#include "k3_topk.h"

namespace k3 {

namespace {

__device__ __forceinline__ double bf16_lo(uint32_t v) {
  return (double)__uint_as_float(v << 16);
}
__device__ __forceinline__ double bf16_hi(uint32_t v) {
  return (double)__uint_as_float(v & 0xFFFF0000u);
}

// acc[j] += products of element pair j of the 8 (4 independent chains).
__device__ __forceinline__ void dot8_bf16(u32x4 a, u32x4 b, double (&acc)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[i] = fma(bf16_lo(a[i]), bf16_lo(b[i]), acc[i]);
    acc[i] = fma(bf16_hi(a[i]), bf16_hi(b[i]), acc[i]);
  }
}

// DPP reductions over the 64 lanes (row_shr 1,2,4,8, then row_bcast 15 and
// 31); the result of lane 63 is returned to every lane. Lanes without a DPP
// source keep their own value.
// Sum over the 64 lanes in a fixed DPP tree (lanes without a source add 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d0(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS,
                                             0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS,
                                             0xf, false);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_d0<0x111, 0xf>(v);
  v += dpp_d0<0x112, 0xf>(v);
  v += dpp_d0<0x114, 0xf>(v);
  v += dpp_d0<0x118, 0xf>(v);
  v += dpp_d0<0x142, 0xa>(v);
  v += dpp_d0<0x143, 0xc>(v);
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  return __hiloint2double(hi, lo);
}

constexpr int kRouterWaves = 4;
constexpr int kRouterCPL = 16;  // 16-byte chunks per lane in flight

__global__ __launch_bounds__(kRouterWaves * 64) void router_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ R, int hidden,
    int n, double *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kRouterWaves + wave_id();
  const int t = blockIdx.y;
  if (e >= n) return;  // whole wave; no barrier below
  gu4_t *Rr = (gu4_t *)(R + (size_t)e * hidden);
  gu4_t *xr = (gu4_t *)(x + (size_t)t * hidden);
  const int nchunk = hidden / 8;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = 0; c0 < nchunk; c0 += 64 * kRouterCPL) {
    // Every lane loads (at a clamped index) so that all loads issue before
    // the first use; lanes past the row's end then use zeros.
    u32x4 rv[kRouterCPL], xv[kRouterCPL];
#pragma unroll
    for (int i = 0; i < kRouterCPL; ++i) {
      if (c0 + 64 * i >= nchunk) break;  // wave-uniform
      const int c = min(c0 + lane + 64 * i, nchunk - 1);
      rv[i] = Rr[c];
      xv[i] = xr[c];
    }
#pragma unroll
    for (int i = 0; i < kRouterCPL; ++i) {
      if (c0 + 64 * i >= nchunk) break;
      const bool ok = c0 + lane + 64 * i < nchunk;
      const u32x4 z = {0u, 0u, 0u, 0u};
      dot8_bf16(ok ? rv[i] : z, ok ? xv[i] : z, acc);
    }
  }
  const double total = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
  if (lane == 0) logits[(size_t)t * n + e] = total;
}


template <int KPL, typename LT>
__global__ __launch_bounds__(64) void topk_kernel(const LT *__restrict__ logits,
                                                  const float *__restrict__ bias,
                                                  int n, int k,
                                                  int32_t *__restrict__ idx,
                                                  float *__restrict__ w) {
  __shared__ TopkLds tk;
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  int sel;
  float wt;
  topk_wave<KPL, LT>(logits + (size_t)t * n, bias, n, k, tk, &sel, &wt);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel;
    w[(size_t)t * k + lane] = wt;
  }
}

template <typename LT>
hipError_t launch_topk(const LT *logits, const float *bias, int T, int n,
                       int k, int32_t *idx, float *w, hipStream_t s) {
  const int kpl = (n + 63) / 64;
#define K3_TOPK_CASE(KPL)                                                      \
  if (kpl <= KPL) {                                                            \
    hipLaunchKernelGGL((topk_kernel<KPL, LT>), dim3(T), dim3(64), 0, s,       \
                       logits, bias, n, k, idx, w);                            \
    return hipGetLastError();                                                  \
  }
  K3_TOPK_CASE(1)
  K3_TOPK_CASE(2)
  K3_TOPK_CASE(4)
  K3_TOPK_CASE(8)
  K3_TOPK_CASE(16)
  K3_TOPK_CASE(32)
  K3_TOPK_CASE(64)
#undef K3_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_router(const uint16_t *x, const uint16_t *R, int T,
                         int hidden, int n, double *logits, hipStream_t s) {
  hipLaunchKernelGGL(router_kernel,
                     dim3((n + kRouterWaves - 1) / kRouterWaves, T),
                     dim3(kRouterWaves * 64), 0, s, x, R, hidden, n, logits);
  return hipGetLastError();
}

hipError_t launch_topk_f64(const double *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s) {
  return launch_topk(logits, bias, T, n, k, idx, w, s);
}

hipError_t launch_topk_f32(const float *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s) {
  return launch_topk(logits, bias, T, n, k, idx, w, s);
}

}  // namespace k3
