// Device-side MXFP4 decode and per-row dot products for gfx950.
//
// Decode uses gfx950's scaled FP4 conversions, which turn the two E2M1 codes
// of one byte into two fp32 (or two bf16) values in a single instruction,
// element 2b from the low nibble; the 16-entry table lives in the hardware
// instead of in memory, so a group of 32 codes costs 16 conversions. The
// group's dot product is accumulated in fp32 and its E8M0 exponent is applied
// once, after the group ([SAT] "Reduction one"): acc += 2^(e-127) * sub, with
// exponent byte 255 skipped by a select so that non-finite activations inside
// such a group cannot reach the row ([A176] "What byte-identical actually
// costs").
//
// Activations are wave-uniform (every lane owns a different row but all lanes
// read the same x group), so the compiler keeps them in scalar registers and
// each VALU operation takes x straight from an SGPR.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k3_internal.h"

namespace k3 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Activation groups are wave-uniform and never written by the kernels that
// read them, so they are read through the constant address space: scalar
// loads into SGPRs that every VALU instruction can take as an operand.
typedef __attribute__((address_space(4))) const uint32_t cu32_t;
typedef __attribute__((address_space(4))) const float cf32_t;

// sum_{i<32} E2M1(code_i) * x_i for x bf16 (16 packed pairs at xg).
__device__ __forceinline__ float group_dot_bf16(const u32x4 w,
                                                const uint32_t *xg) {
  const cu32_t *xc = (const cu32_t *)xg;
  float s = 0.f;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const bf16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 0);
    const bf16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 1);
    const bf16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 2);
    const bf16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 3);
    s = __builtin_amdgcn_fdot2_f32_bf16(w0, __builtin_bit_cast(bf16x2, xc[4 * d + 0]), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w1, __builtin_bit_cast(bf16x2, xc[4 * d + 1]), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w2, __builtin_bit_cast(bf16x2, xc[4 * d + 2]), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w3, __builtin_bit_cast(bf16x2, xc[4 * d + 3]), s, false);
  }
  return s;
}

// sum_{i<32} E2M1(code_i) * x_i for x fp32 (32 values at xg).
__device__ __forceinline__ float group_dot_f32(const u32x4 w, const float *xg) {
  const cf32_t *xc = (const cf32_t *)xg;
  float s = 0.f;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 3);
    s = fmaf(v0.x, xc[8 * d + 0], s);
    s = fmaf(v0.y, xc[8 * d + 1], s);
    s = fmaf(v1.x, xc[8 * d + 2], s);
    s = fmaf(v1.y, xc[8 * d + 3], s);
    s = fmaf(v2.x, xc[8 * d + 4], s);
    s = fmaf(v2.y, xc[8 * d + 5], s);
    s = fmaf(v3.x, xc[8 * d + 6], s);
    s = fmaf(v3.y, xc[8 * d + 7], s);
  }
  return s;
}

// A group's 32 codes decoded once, for multiplying by several activation
// vectors: 16 bf16 pairs (exact) or 16 fp32 pairs, element 2i+0 first.
struct GroupBf16 {
  bf16x2 v[16];
};
struct GroupF32 {
  f32x2 v[16];
};

__device__ __forceinline__ GroupBf16 decode_bf16(const u32x4 w) {
  GroupBf16 G;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    G.v[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 0);
    G.v[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 1);
    G.v[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 2);
    G.v[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 3);
  }
  return G;
}

__device__ __forceinline__ GroupF32 decode_f32(const u32x4 w) {
  GroupF32 G;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    G.v[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 0);
    G.v[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 1);
    G.v[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 2);
    G.v[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 3);
  }
  return G;
}

// sum over the group of decoded weights times bf16 x (16 pairs at xg), in
// the same order as group_dot_bf16.
__device__ __forceinline__ float dot_decoded(const GroupBf16 &G,
                                             const uint32_t *xg) {
  const cu32_t *xc = (const cu32_t *)xg;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    s = __builtin_amdgcn_fdot2_f32_bf16(G.v[i], __builtin_bit_cast(bf16x2, xc[i]), s, false);
  return s;
}

// Same for fp32 x (32 values at xg), in the order of group_dot_f32.
__device__ __forceinline__ float dot_decoded(const GroupF32 &G, const float *xg) {
  const cf32_t *xc = (const cf32_t *)xg;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s = fmaf(G.v[i].x, xc[2 * i], s);
    s = fmaf(G.v[i].y, xc[2 * i + 1], s);
  }
  return s;
}

// acc += 2^(e-127) * sub, or nothing for e == 255 (select, not multiply).
__device__ __forceinline__ float apply_scale(float acc, float sub, uint32_t e) {
  const float t = acc + ldexpf(sub, (int)e - 127);
  return e == 255u ? acc : t;
}

// Global-address-space views, so loads through pointers read from device
// memory (e.g. an expert table) compile to global_load rather than flat_load.
typedef __attribute__((address_space(1))) const u32x4 gu4_t;
typedef __attribute__((address_space(1))) const uint32_t gu32_t;

// Wave-uniform read of data the kernel never writes, through the constant
// address space: a scalar load (counted by lgkmcnt), so it never makes the
// weight stream's vector-load waits conservative.
template <typename T>
__device__ __forceinline__ T ldc(const T *p) {
  return *(const __attribute__((address_space(4))) T *)p;
}

#ifndef K3_NW
#define K3_NW 16
#endif
constexpr int kNW = K3_NW;   // waves per workgroup of the streaming kernels
constexpr int kMaxTPW = 8;   // tiles per pass of one workgroup

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Contiguous tile range of workgroup b out of `grid` for `total` tiles.
__device__ __forceinline__ void wg_range(int total, int *t0, int *t1) {
  const long long b = blockIdx.x, n = gridDim.x;
  *t0 = (int)(b * total / n);
  *t1 = (int)((b + 1) * total / n);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace k3
