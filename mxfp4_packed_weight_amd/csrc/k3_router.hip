// Router: bf16 logits GEMV in fp64 and sigmoid top-k selection.
//
// Logits: four waves per (token, expert) row (router_row_part, k3_router.h:
// all of a row's loads in flight at once, fp64 products and sums in a fixed
// order, reproducible bit for bit).
//
// Selection: one wave per token with the keys in registers; a cheap lower
// bound keeps ~18 candidates, which are ranked in parallel (topk_wave,
// k3_topk.h). Ties go to the lower expert index. The routing bias only
// changes the keys; the weights always come from the unbiased sigmoid scores
// ([ZOR] "How is the C engine actually built?", invariant 3), renormalised to
// sum to one, summed in rank order.
#include <limits.h>
#include <math.h>

#include "k3_router.h"
#include "k3_topk.h"

namespace k3 {

namespace {

// One workgroup of kRouterSplit waves per (row, token); tokens beyond the
// grid's y extent are taken in strides of it.
static_assert(kRouterSplit == 4, "the partials are added as (p0 + p1) + (p2 + p3)");
// NT: one token (each router row is read once, non-temporally).
template <bool NT>
__global__ __launch_bounds__(kRouterSplit * 64) void router_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ R, int hidden,
    int n, int T, double *__restrict__ logits) {
  __shared__ double partial[kRouterSplit];
  const int e = blockIdx.x;
  for (int t = blockIdx.y; t < T; t += gridDim.y)
    router_row_logit<NT>(R + (size_t)e * hidden, x + (size_t)t * hidden, hidden, partial,
                         logits + (size_t)t * n + e);
}


template <int KPL, typename LT>
__global__ __launch_bounds__(64) void topk_kernel(const LT *__restrict__ logits,
                                                  const float *__restrict__ bias,
                                                  int n, int k,
                                                  int32_t *__restrict__ idx,
                                                  float *__restrict__ w, double scale) {
  __shared__ TopkLds tk;
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  int sel;
  float wt;
  topk_wave<KPL, LT>(logits + (size_t)t * n, bias, n, k, tk, &sel, &wt, scale);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel;
    w[(size_t)t * k + lane] = wt;
  }
}

template <typename LT>
hipError_t launch_topk(const LT *logits, const float *bias, int T, int n,
                       int k, int32_t *idx, float *w, hipStream_t s,
                       double scale = 1.0) {
  const int kpl = (n + 63) / 64;
#define K3_TOPK_CASE(KPL)                                                      \
  if (kpl <= KPL) {                                                            \
    hipLaunchKernelGGL((topk_kernel<KPL, LT>), dim3(T), dim3(64), 0, s,       \
                       logits, bias, n, k, idx, w, scale);                     \
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
  if (T == 1)
    hipLaunchKernelGGL(router_kernel<true>, dim3(n, 1), dim3(kRouterSplit * 64), 0, s, x, R,
                       hidden, n, T, logits);
  else
    hipLaunchKernelGGL(router_kernel<false>, dim3(n, T < 65535 ? T : 65535),
                       dim3(kRouterSplit * 64), 0, s, x, R, hidden, n, T, logits);
  return hipGetLastError();
}

hipError_t launch_topk_f64(const double *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s, double scale) {
  return launch_topk(logits, bias, T, n, k, idx, w, s, scale);
}

hipError_t launch_topk_f32(const float *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s) {
  return launch_topk(logits, bias, T, n, k, idx, w, s);
}

}  // namespace k3
