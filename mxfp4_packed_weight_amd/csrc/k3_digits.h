// The single-token MXFP4 product on the matrix unit: a 64-row tile of packed
// E2M1 codes times one activation vector, with the codes fed to the
// instruction as they are stored (no decode to floats on the vector ALU).
//
// Instruction: v_mfma_scale_f32_16x16x128_f8f6f4 with A = the codes (FP4,
// E2M1) and B = the activations (FP8, E4M3), every 32-element K block of
// either operand scaled by an E8M0 exponent of its own, so the weights'
// exponent bytes (one per 32 weights of a row, [A176] "The four reductions")
// are the A scales unchanged.
//
// Operand layouts (measured on gfx950):
//   A (FP4): lane l = row l%16, K [32(l/16), +32): 16 bytes, the low nibble
//            first, i.e. one 32-code group of one row; its scale is that
//            group's exponent byte.
//   B (FP8): lane l = column l%16, bytes 0..15 = K [16(l/16), +16) and bytes
//            16..31 = K [64 + 16(l/16), +16); the scale held by lane l is
//            that of column l%16's K block [32(l/16), +32).
//   C:       lane l = column l%16, rows 4(l/16) + i, i = 0..3.
// A quad of the tile layout (lane r = row r, its four 16-byte registers =
// groups 4q..4q+3) becomes the A operands of row blocks m = 0..3 by a 4 x 4
// transpose of (register, 16-lane row), two v_permlane32_swap and two
// v_permlane16_swap per dword; the exponent bytes go through the same
// transpose. One instruction per 16-row block and quad: four per quad.
//
// Activation digits. The instruction adds a K block's 32 products exactly
// only while they span less than about 2^8 (measured: activations rounded to
// FP8 gave errors of 1e-5 of the output), so activations are not rounded to
// FP8. Each group of 32 values is cut into kDigits fixed-point slices of 4
// bits below the group's largest exponent Emax:
//   v = sum_{p < kDigits} d_p 2^(Emax - 3 - 4p) + r,
// the d_p in [-15, 15] the base-16 digits of |v| rounded to nearest (ties to
// even) at 2^(Emax - 23), with v's sign, so |r| <= 2^(Emax - 24). Slice p is
// B column p. The E4M3 code of a digit is the digit itself (sign in bit 7):
// codes 0..7 are the subnormals m 2^-9 and codes 8..15 the values
// (8 + m) 2^-9 of the first binade, so code d means d 2^-9 exactly and the
// slice's block exponent is Emax - 3 - 4p + 9. A block's products code * d_p
// span at most 6 * 15 / 0.5 < 2^8, so each block sum is exact (measured with
// these codes as well). A bf16 value within 2^-16 of its group's largest is
// carried exactly, any other value to within half an fp32 ulp of the
// group's largest (fp32's own rounding of a sum that holds it). Columns
// kDigits..15 repeat the last slice and are ignored; a row's result is the
// sum of its kDigits columns, smallest slice first.
//
// Exponent bytes. Byte 255 makes its group contribute nothing ([A176] "What
// byte-identical actually costs"): a quad that holds one gets that group's
// codes zeroed and a finite scale in the lanes concerned before it is
// multiplied. Every other byte is the instruction's scale as it stands, so
// results outside [2, 252] follow fp32 range as the vector-ALU route's do.
//
// Vector-ALU route. Activation groups that hold a non-finite value, or whose
// largest value is below 2^-87 or at least 2^122 (beyond the range of the
// slice exponents), are flagged when the digits are built; a
// workgroup whose vectors have a flagged group (or do not fit in its LDS)
// streams its tiles on the vector ALU instead, group by group as in
// k3_decode.h. The choice is made once per workgroup, before any quad is
// multiplied, so each loop holds only one route's code.
#pragma once

#include "k3_decode.h"

namespace k3 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

constexpr int kDigits = 6;                      // slices per activation group
constexpr int kSliceQuadBytes = kDigits * 128;  // one quad's slices
constexpr int kGroupMeta = 8;                   // per group: 6 slice exponents, flag, 0
constexpr int kDigitQuadBytes = kSliceQuadBytes + 4 * kGroupMeta;
constexpr int kMaxDigitQuads = K3_MAX_HIDDEN / 128;
constexpr int kDigitLds = kMaxDigitQuads * kDigitQuadBytes;  // LDS per kernel
static_assert(kDigitQuadBytes % 16 == 0, "vectors stay 16-byte aligned");

// Digits of one activation vector of G4 quads (a multiple of 16 bytes):
//   [G4][kDigits][128]  slice p of quad q: its 128 values in K order
//   [4 G4][8]           per group: exponent byte of slices 0..5, flag, 0
__host__ __device__ inline int digit_bytes(int G4) { return G4 * kDigitQuadBytes; }
__host__ __device__ inline int digit_meta_off(int G4) { return G4 * kSliceQuadBytes; }

// |v| in units of 2^(Emax - 23), rounded to nearest (ties to even): the 24
// bits that the group's six 4-bit slices hold. u = v's fp32 bits; unit =
// 2^(23 - Emax) = 2^(150 - emax) for the group's largest exponent field emax
// (a normal float for the groups that are not flagged). The product is
// exact and below 2^24, so rint gives the integer exactly.
__device__ __forceinline__ uint32_t digit_mag(uint32_t u, float unit) {
  return (uint32_t)rintf(__uint_as_float(u & 0x7FFFFFFFu) * unit);
}
__device__ __forceinline__ float digit_unit(uint32_t emax) {
  return __uint_as_float((277u - emax) << 23);
}

// Largest of v over the four lanes of this lane's DPP quad: the four lanes
// that hold one activation group.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // lane ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // lane ^ 2
  return v;
}

// The eight meta bytes of a group from m, the fp32 bits of its largest
// magnitude (its largest exponent field is m >> 23, as magnitudes order like
// their bits): the slice exponent bytes (Emax - 3 - 4p + 9) + 127 =
// emax + 6 - 4p for p = 0..5, a flag byte, 0. Flagged: a non-finite value,
// or a non-zero group whose emax is outside [40, 248]. A flagged or all-zero
// group gets exponent bytes 127.
__device__ __forceinline__ void group_meta(uint32_t m, uint32_t &lo4, uint32_t &hi4) {
  const uint32_t emax = m >> 23;
  const bool flag = emax > 248u || (m != 0u && emax < 40u);
  const bool live = !flag && m != 0u;
  // emax + 6 in all four bytes; no byte borrows below, as emax + 6 >= 46
  const uint32_t e4 = __builtin_amdgcn_perm(0u, emax + 6u, 0u);
  lo4 = live ? e4 - 0x0C080400u : 0x7F7F7F7Fu;
  hi4 = live ? (e4 & 0xFFFFu) - 0x1410u : (flag ? 0x17F7Fu : 0x7F7Fu);
}

// Building the digits of one activation vector of G groups (G4 quads in the
// buffer; groups past G get zero digits and finite exponents). Four lanes
// per group (one DPP quad), eight values each: task t of the vector is
// values [8t, 8t + 8), quarter t & 3 of group t >> 2; thread i takes tasks
// i, i + kDigitThreads, ... Every thread of the workgroup (kNW waves) takes
// part. The loads are a step of their own so that a caller can issue them
// early and do the arithmetic while other loads are in flight.
constexpr int kDigitThreads = kNW * 64;
constexpr int kDigitTasks = (kMaxDigitQuads * 16 + kDigitThreads - 1) / kDigitThreads;

// This thread's tasks as loaded: eight fp32 (W = 8) or eight bf16 packed in
// pairs, the lower half first (W = 4).
template <int W>
struct DigitFetch {
  uint32_t r[kDigitTasks][W];
  // fp32 bits of value i of pass k
  __device__ __forceinline__ uint32_t bits(int k, int i) const {
    if constexpr (W == 8) return r[k][i];
    return (i & 1) ? (r[k][i >> 1] & 0xFFFF0000u) : (r[k][i >> 1] << 16);
  }
  // sign bits of values 4h..4h+3 of pass k, in bit 7 of bytes 0..3
  __device__ __forceinline__ uint32_t signs(int k, int h) const {
    uint32_t s;
    if constexpr (W == 8)
      s = __builtin_amdgcn_perm(r[k][4 * h + 1], r[k][4 * h], 0x0C0C0703u) |
          __builtin_amdgcn_perm(r[k][4 * h + 3], r[k][4 * h + 2], 0x07030C0Cu);
    else
      s = __builtin_amdgcn_perm(r[k][2 * h + 1], r[k][2 * h], 0x07050301u);
    return s & 0x80808080u;
  }
};

// Step one: load(t, r) fills r[0..W) with task t's values (t < 4 G).
template <int W, class Load>
__device__ __forceinline__ void fetch_digits(Load load, int G, DigitFetch<W> &f) {
#pragma unroll
  for (int k = 0; k < kDigitTasks; ++k) {
    const int task = (int)threadIdx.x + k * kDigitThreads;
    if (task < 4 * G) {
      load(task, f.r[k]);
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) f.r[k][i] = 0u;
    }
  }
}

// Step two: the digits into dst. Returns (per thread) whether this thread
// wrote a flagged group; the caller synchronises before the digits are read.
// A flagged group's digit bytes are left undefined: its workgroup streams
// on the vector ALU and never reads them.
template <int W>
__device__ __forceinline__ bool compute_digits(const DigitFetch<W> &f, int G4, lds_u8 *dst) {
  const int n = 16 * G4;  // tasks, those of the padding groups included
  bool flagged = false;
#pragma unroll
  for (int k = 0; k < kDigitTasks; ++k) {
    if (k * kDigitThreads >= n) break;  // uniform
    const int task = (int)threadIdx.x + k * kDigitThreads, gi = task >> 2, a = task & 3;
    uint32_t u[8], m = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u[i] = f.bits(k, i);
      m = max(m, u[i] & 0x7FFFFFFFu);
    }
    m = quad_max(m);
    if (task >= n) continue;
    uint32_t lo4, hi4;
    group_meta(m, lo4, hi4);  // a group past G reads as all zero
    // finite for every group that is not flagged; a zero group's values
    // give zero digits with it
    const float unit = digit_unit(m >> 23);
    uint32_t F[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) F[i] = digit_mag(u[i], unit);
    const int q = gi >> 2, j = gi & 3;
    lds_u8 *sl = dst + q * kSliceQuadBytes + 32 * j + 8 * a;
    uint32_t S[kDigits][2];  // slice p, values 4h..4h+3
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t sgn = f.signs(k, h);
#pragma unroll
      for (int kb = 2; kb >= 0; --kb) {  // byte kb of the 24 bits: slices 4 - 2kb, 5 - 2kb
        const uint32_t sel = (uint32_t)kb | ((uint32_t)(4 + kb) << 8) | 0x0C0C0000u;
        const uint32_t Bk = __builtin_amdgcn_perm(F[4 * h + 1], F[4 * h], sel) |
                            (__builtin_amdgcn_perm(F[4 * h + 3], F[4 * h + 2], sel) << 16);
        S[4 - 2 * kb][h] = ((Bk >> 4) & 0x0F0F0F0Fu) | sgn;
        S[5 - 2 * kb][h] = (Bk & 0x0F0F0F0Fu) | sgn;
      }
    }
#pragma unroll
    for (int p = 0; p < kDigits; ++p) {
      lds_u32 *d = (lds_u32 *)(sl + p * 128);
      d[0] = S[p][0];
      d[1] = S[p][1];
    }
    if (a == 0) {
      lds_u32 *meta = (lds_u32 *)(dst + digit_meta_off(G4) + kGroupMeta * gi);
      meta[0] = lo4;
      meta[1] = hi4;
    }
    flagged |= (hi4 >> 16) != 0u;
  }
  return flagged;
}

// Both steps at once, for a vector loaded one value at a time: load(i) is
// element i as an exact fp32 value.
template <class Load>
__device__ __forceinline__ bool build_digits(Load load, int G, int G4, lds_u8 *dst) {
  DigitFetch<8> f;
  fetch_digits<8>(
      [&](int t, uint32_t(&r)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = __float_as_uint(load(8 * t + i));
      },
      G, f);
  return compute_digits(f, G4, dst);
}

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// Copies n bytes (a multiple of 4) from src (device memory, 4-byte aligned)
// to dst (LDS) without registers: the wave's lanes load dwords straight into
// LDS. The copies count as vector loads of the issuing wave, so a wave's
// vmcnt(0) wait covers its own; a barrier after every wave's wait covers all.
__device__ __forceinline__ void dma_to_lds(const uint8_t *src, lds_u8 *dst, int n) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  for (int c = wave * 256; c < n; c += kNW * 256)
    if (c + 4 * lane < n)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(src + c + 4 * lane), (lvoid_t *)(dst + c), 4,
                                       0, 0);
}

// Digits of a bf16 vector of G groups already copied to LDS (xs, 2 bytes
// per value, 16-byte aligned) into dst; as compute_digits.
__device__ __forceinline__ bool compute_digits_bf16(const lds_u8 *xs, int G, int G4,
                                                    lds_u8 *dst) {
  DigitFetch<4> f;
  fetch_digits<4>(
      [&](int t, uint32_t(&r)[4]) {
        const u32x4 v = ((const lds_u4 *)xs)[t];
        r[0] = v[0];
        r[1] = v[1];
        r[2] = v[2];
        r[3] = v[3];
      },
      G, f);
  return compute_digits(f, G4, dst);
}

// 4 x 4 transpose of (register, 16-lane row): afterwards register m of lane
// row j holds what register j of lane row m held.
__device__ __forceinline__ void transpose4(uint32_t &r0, uint32_t &r1, uint32_t &r2,
                                           uint32_t &r3) {
  const auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

// This lane's fixed offsets into a digit buffer: its B bytes (slice
// min(l%16, kDigits - 1), K rows 16(l/16)..) and its scale byte (group l/16
// of a quad, same slice).
struct DigitLane {
  int b_off, s_off;
};
__device__ __forceinline__ DigitLane digit_lane() {
  const int l = threadIdx.x & 63, g = l >> 4, c = min(l & 15, kDigits - 1);
  return DigitLane{c * 128 + 16 * g, g * kGroupMeta + c};
}

// acc[m] += rows 16m..16m+15 of quad q times the digits D (G4 quads): w and e
// are this lane's registers of the quad (row = lane). Groups whose exponent
// byte is 255 contribute nothing: their codes are zeroed and their scale
// made finite first (only in a quad that has one).
__device__ __forceinline__ void mx_quad(const u32x4 (&w)[4], uint32_t e, const lds_u8 *D, int G4,
                                        int q, DigitLane dl, f32x4 (&acc)[4]) {
  uint32_t r[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    r[b][0] = w[b].x;
    r[b][1] = w[b].y;
    r[b][2] = w[b].z;
    r[b][3] = w[b].w;
  }
  const uint32_t ff = ((e & 0x7F7F7F7Fu) + 0x01010101u) & e & 0x80808080u;  // bytes == 255
  if (__builtin_amdgcn_ballot_w64(ff != 0u) != 0u) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if ((ff >> (8 * b + 7)) & 1u) r[b][0] = r[b][1] = r[b][2] = r[b][3] = 0u;
    e &= ~((ff >> 7) * 0xFFu);
  }
  uint32_t s[4] = {e & 255u, (e >> 8) & 255u, (e >> 16) & 255u, e >> 24};
#pragma unroll
  for (int d = 0; d < 4; ++d) transpose4(r[0][d], r[1][d], r[2][d], r[3][d]);
  transpose4(s[0], s[1], s[2], s[3]);
  const lds_u8 *qb = D + q * kSliceQuadBytes + dl.b_off;
  const u32x4 lo = *(const lds_u4 *)qb, hi = *(const lds_u4 *)(qb + 64);
  const int sb = D[digit_meta_off(G4) + q * 4 * kGroupMeta + dl.s_off];
  const v8i B = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const v8i A = {(int)r[m][0], (int)r[m][1], (int)r[m][2], (int)r[m][3], 0, 0, 0, 0};
    acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[m], 4, 0, 0, (int)s[m],
                                                              0, sb);
  }
}

// Value of lane + K (same 16-lane row) for lanes whose l%16 + K < 16.
template <int K>
__device__ __forceinline__ float from_lane_plus(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + K, 0xF, 0xF, true));
}

// Finishes a row tile's partial: out[r] (LDS, 64 floats) = the sum of row r's
// kDigits columns, smallest slice first. acc is reset.
__device__ __forceinline__ void mx_flush(f32x4 (&acc)[4], float *out) {
  static_assert(kDigits == 6, "the column sum below is written out for six slices");
  const int l = threadIdx.x & 63, g = l >> 4;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f32x4 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = acc[m][i];
      float t = from_lane_plus<5>(v);
      t += from_lane_plus<4>(v);
      t += from_lane_plus<3>(v);
      t += from_lane_plus<2>(v);
      t += from_lane_plus<1>(v);
      s[i] = t + v;
    }
    if ((l & 15) == 0) *reinterpret_cast<f32x4 *>(out + 16 * m + 4 * g) = s;
    acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

}  // namespace k3
