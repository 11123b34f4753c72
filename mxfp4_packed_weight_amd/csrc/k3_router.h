// One router row's logit: bf16 x . bf16 R[e] with every product and sum in
// fp64, split over kRouterSplit waves.
//
// Each lane issues the loads of all its 16-byte chunks of the row before
// computing, so a whole row is in flight at once; products go into four
// chains per lane ((0 + 1) + (2 + 3) at the end), the lane sums are combined
// by a fixed DPP tree and the waves' partials in a fixed order. A product of
// two bf16 values is exact in fp64, so a logit is within ~1e-16 of a
// sequential fp64 sum, which keeps the top-k indices identical to an fp64
// reference.
#pragma once

#include "k3_decode.h"

namespace k3 {

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

constexpr int kRouterCPL = 8;  // 16-byte chunks per lane in flight
constexpr int kRouterSplit = 4;  // waves per router row

// This wave's share of one router row's logit: wave `part` of kRouterSplit
// takes chunks c = 64 (kRouterSplit i + part) + lane, x from global memory
// (XLds = false, at xg) or from the workgroup's LDS copy (XLds = true, at
// xl); R row at Rrow; hidden a multiple of 8. Returns the wave's fp64 sum
// (four chains per lane, then the DPP tree), the same in every lane; the
// kRouterSplit partials are added as (p0 + p1) + (p2 + p3). NT: the row is
// read once (one token), so its loads are non-temporal; with several tokens
// the row is read once per token and stays cached.
template <bool XLds, bool NT>
__device__ __forceinline__ double router_row_part(const uint16_t *__restrict__ Rrow,
                                                  const uint16_t *__restrict__ xg,
                                                  const u32x4 *xl, int hidden,
                                                  int part) {
  const int lane = threadIdx.x & 63;
  gu4_t *Rr = (gu4_t *)Rrow;
  gu4_t *xr = (gu4_t *)xg;
  const int nchunk = hidden / 8;
  constexpr int kStride = 64 * kRouterSplit;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = 64 * part; c0 < nchunk; c0 += kStride * kRouterCPL) {
    // Every lane loads (at a clamped index) so that all loads issue before
    // the first use; lanes past the row's end then use zeros.
    u32x4 rv[kRouterCPL], xv[kRouterCPL];
#pragma unroll
    for (int i = 0; i < kRouterCPL; ++i) {
      if (c0 + kStride * i >= nchunk) break;  // wave-uniform
      const int c = min(c0 + lane + kStride * i, nchunk - 1);
      rv[i] = NT ? __builtin_nontemporal_load(Rr + c) : Rr[c];
      if (!XLds) xv[i] = xr[c];
    }
#pragma unroll
    for (int i = 0; i < kRouterCPL; ++i) {
      if (c0 + kStride * i >= nchunk) break;
      const int c = c0 + lane + kStride * i;
      const bool ok = c < nchunk;
      if (XLds) xv[i] = xl[min(c, nchunk - 1)];
      const u32x4 z = {0u, 0u, 0u, 0u};
      dot8_bf16(ok ? rv[i] : z, ok ? xv[i] : z, acc);
    }
  }
  return wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
}

// Logit of router row e for token x: the kRouterSplit waves of the
// calling workgroup each take their part and wave 0's lane 0 stores
// (p0 + p1) + (p2 + p3). `partial` is the workgroup's LDS scratch.
template <bool NT>
__device__ __forceinline__ void router_row_logit(const uint16_t *__restrict__ Rrow,
                                                 const uint16_t *__restrict__ x,
                                                 int hidden, double *partial,
                                                 double *out) {
  const int w = wave_id();
  const double p = router_row_part<false, NT>(Rrow, x, nullptr, hidden, w);
  if ((threadIdx.x & 63) == 0) partial[w] = p;
  __syncthreads();
  if (threadIdx.x == 0) *out = (partial[0] + partial[1]) + (partial[2] + partial[3]);
  __syncthreads();
}

}  // namespace k3
