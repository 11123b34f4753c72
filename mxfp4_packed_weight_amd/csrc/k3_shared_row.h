// One output row of the shared experts' down stage, used by the separate
// shared-down launch and by the decode layer's expert launch, which takes
// the rows between its gate/up and down stages. The same code in both gives
// the same bits.
#pragma once

#include "k3_decode.h"

namespace k3 {

__device__ __forceinline__ float lanes_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));

// 16 bytes read once (non-temporal).
__device__ __forceinline__ uint4 ld16_nt(const uint16_t *p) {
  const u32v4 v = __builtin_nontemporal_load(reinterpret_cast<const u32v4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ys[r] = sum over s of W_down(s)[r] . h[s], by one wave (the result in every
// lane): lane l takes columns 8l + 512m of every shared expert in turn (s
// ascending, then m ascending), then the lanes are summed. Blob of shared
// expert s: gate [inter][hidden], up [inter][hidden], down [hidden][inter],
// bf16 row-major; h [n_shared][inter] fp32.
__device__ __forceinline__ float shared_down_row(const float *__restrict__ h,
                                                 const uint16_t *const *__restrict__ shared,
                                                 int n_shared, int hidden, int inter, int r) {
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int s = 0; s < n_shared; ++s) {
    const uint16_t *dr = shared[s] + (size_t)2 * inter * hidden + (size_t)r * inter;
    const float4 *hv = reinterpret_cast<const float4 *>(h + (size_t)s * inter);
#pragma unroll 2
    for (int c8 = lane; 8 * c8 < inter; c8 += 64) {
      const uint4 w = ld16_nt(dr + 8 * c8);
      const float4 h0 = hv[2 * c8], h1 = hv[2 * c8 + 1];
      acc = fmaf(__uint_as_float(w.x << 16), h0.x, acc);
      acc = fmaf(__uint_as_float(w.x & 0xFFFF0000u), h0.y, acc);
      acc = fmaf(__uint_as_float(w.y << 16), h0.z, acc);
      acc = fmaf(__uint_as_float(w.y & 0xFFFF0000u), h0.w, acc);
      acc = fmaf(__uint_as_float(w.z << 16), h1.x, acc);
      acc = fmaf(__uint_as_float(w.z & 0xFFFF0000u), h1.y, acc);
      acc = fmaf(__uint_as_float(w.w << 16), h1.z, acc);
      acc = fmaf(__uint_as_float(w.w & 0xFFFF0000u), h1.w, acc);
    }
  }
  return lanes_sum(acc);
}

}  // namespace k3
