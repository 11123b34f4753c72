// Matrix-vector products on gfx950's block-scaled FP4 matrix instruction.
//
// The weights stay packed: every 16-byte lane load of a tile (see
// k3_internal.h) is one 32-code MXFP4 group, and a 1 KiB sub-block is the A
// operand of v_mfma_scale_f32_16x16x128_f8f6f4 with the groups' E8M0
// exponents as the A scales, so the E2M1 table and the power-of-two scale
// are applied by the matrix unit itself and the product is never expanded
// to floats in memory ([SAT] "Reduction one").
//
// The activation vector is the B operand, split into P exact fixed-point
// E4M3 "pieces" (B columns 0..P-1; the other columns are zero). For every
// block of 32 elements with largest magnitude in [2^e, 2^(e+1)), piece c is
// the residual rounded to the grid 2^(e-3-5c): an integer in [-16, 16]
// (exact in E4M3) under the E8M0 exponent e-3-5c, the B scale of that block
// and column. Summing the P output columns gives W x; five pieces leave a
// residual below 2^-24 of the block maximum, the size of fp32 rounding.
// Fixed point matters: the matrix unit aligns the products of a block to
// its largest one and keeps about 13 bits below it (measured on MI355X), so
// the pieces are kept within 2^5 of each other and every product of a block
// (E2M1 x integer <= 16) is exact; block sums are added with fp32 precision.
//
// Operand layouts (measured on MI355X, 16x16x128, A = FP4, B = FP8 E4M3):
//   A: lane l = row l%16, K elements [32(l/16), +32), low nibble = even k;
//   B: lane l = column l%16, K [16(l/16), +16) in bytes 0..15 and
//      [64 + 16(l/16), +16) in bytes 16..31;
//   scales: byte `opsel` of the lane's scale register; A: (row l%16, block
//      l/16), B: (block l/16, column l%16);
//   C: lane l = column l%16, rows 4(l/16) + i, i = 0..3.
// An exponent byte of 255 makes the matrix unit return NaN for the whole
// row, so such groups are zeroed before the product (their contribution is
// exactly zero whenever the activations are finite); calls whose
// activations hold a non-finite value take the VALU path instead, which
// skips 255 groups outright ([A176] "What byte-identical actually costs").
#pragma once

#include "k3_decode.h"
#include "k3_internal.h"

namespace k3 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---- activation pieces -------------------------------------------------
// Compact B fragment of one 128-element K block for P pieces:
//   bytes [32*(h*P + c), +32)  lane (h, c) of the B operand, h = l/16,
//                              c = l%16 < P (lanes c >= P are zero);
//   byte  128*P + kb*P + c     E8M0 exponent of block kb, piece c.
__host__ __device__ constexpr int frag_bytes(int P) {
  return 128 * P + ((4 * P + 15) / 16) * 16;
}
// Integer q in [-16, 16] (held exactly in a float) -> its E4M3 code.
__device__ __forceinline__ uint32_t e4m3_small_int(float q) {
  const uint32_t b = __float_as_uint(fabsf(q));
  if (b == 0u) return 0u;
  const uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);  // biased 127 -> 7
  return q < 0.f ? (code | 0x80u) : code;
}

// Max over the 32 lanes of each wave half; every lane gets its half's max.
__device__ __forceinline__ float halfwave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                   __float_as_int(v), __float_as_int(v), 0x111, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                   __float_as_int(v), __float_as_int(v), 0x112, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                   __float_as_int(v), __float_as_int(v), 0x114, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                   __float_as_int(v), __float_as_int(v), 0x118, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(
                   __float_as_int(v), __float_as_int(v), 0x142, 0xa, 0xf, false)));
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return (threadIdx.x & 32) ? hi : lo;
}

// Pieces of one element: residual r on the grids 2^(e-3-5c), c = 0..P-1,
// with the exponents clamped at -126 (a block below 2^-120 loses what lies
// under 2^-127). Writes the codes to slot[32*c] and the exponent bytes.
template <int P>
__device__ __forceinline__ void split_pieces(float r, float m, uint8_t *slot,
                                             uint8_t *sc, bool write_sc) {
  const int e = (int)((__float_as_uint(m) >> 23) & 255u) - 127;  // m = 0 -> -127
#pragma unroll
  for (int c = 0; c < P; ++c) {
    const int s = max(-126, e - 3 - 5 * c);
    const float q = rintf(r * __uint_as_float((uint32_t)(127 - s) << 23));
    r -= q * __uint_as_float((uint32_t)(127 + s) << 23);
    slot[32 * c] = (uint8_t)e4m3_small_int(q);
    if (write_sc) sc[c] = (uint8_t)(s + 127);
  }
}

// One wave builds the B fragment of one K block. This lane holds elements
// k = lane (block lane/32) and k = lane + 64 (block 2 + lane/32), zero past
// the vector's end; both land in B lane (lane/16, c), bytes lane%16 and
// 16 + lane%16. Every byte the loads read is written. Returns true
// (wave-uniform) if an element is not finite; the fragment is then not
// written.
template <int P>
__device__ __forceinline__ bool make_frag(float v0, float v1, uint8_t *frag,
                                          int lane) {
  const bool bad = !(isfinite(v0) && isfinite(v1));
  if (__ballot(bad)) return true;
  const float m0 = halfwave_max(fabsf(v0)), m1 = halfwave_max(fabsf(v1));
  const int h = lane >> 4, kb0 = lane >> 5, kb1 = 2 + (lane >> 5);
  uint8_t *slot = frag + 32 * h * P + (lane & 15);
  const bool w = (lane & 31) == 0;
  split_pieces<P>(v0, m0, slot, frag + 128 * P + kb0 * P, w);
  split_pieces<P>(v1, m1, slot + 16, frag + 128 * P + kb1 * P, w);
  return false;
}

// ---- fragment building ------------------------------------------------
// A workgroup builds the fragments of nfb 128-element blocks into LDS; wave
// w takes blocks w, w + kNW, ... The activations of its first kPreBlocks
// blocks are loaded ahead, before the first weight loads, so that waiting
// for them does not wait for weights. at(fb, k) must load unconditionally
// (clamped address) so the compiler's load counts stay exact.
constexpr int kPreBlocks = 8;
struct ActPre {
  float v[2 * kPreBlocks];
};

template <class At>
__device__ __forceinline__ ActPre preload_acts(At at, int nfb) {
  const int lane = threadIdx.x & 63, w = wave_id();
  ActPre st;
#pragma unroll
  for (int i = 0; i < kPreBlocks; ++i) {
    const int fb = min(w + kNW * i, nfb - 1);
    st.v[2 * i] = at(fb, lane);
    st.v[2 * i + 1] = at(fb, lane + 64);
  }
  return st;
}

// dst(fb) -> uint8_t*  LDS fragment of block fb. True if a value is not finite.
template <int P, class At, class Dst>
__device__ __forceinline__ bool build_frags(const ActPre &st, At at, int nfb,
                                            Dst dst) {
  const int lane = threadIdx.x & 63, w = wave_id();
  bool bad = false;
#pragma unroll
  for (int i = 0; i < kPreBlocks; ++i)
    if (w + kNW * i < nfb)
      bad |= make_frag<P>(st.v[2 * i], st.v[2 * i + 1], dst(w + kNW * i), lane);
  for (int fb = w + kNW * kPreBlocks; fb < nfb; fb += kNW)
    bad |= make_frag<P>(at(fb, lane), at(fb, lane + 64), dst(fb), lane);
  return bad;
}

// ---- streaming loop ----------------------------------------------------
#ifndef K3_MFMA_DEPTH
#define K3_MFMA_DEPTH 2
#endif
constexpr int kMfmaDepth = K3_MFMA_DEPTH;
constexpr int kPartFloats = kMaxTPW * kNW * 64;  // per-wave row partials
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left free (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// B operand of K block q for this lane from a P-piece fragment array in LDS.
// Lanes of columns >= P read column 0 (so that every lane issues the same
// reads) and then take zeros.
template <int P>
__device__ __forceinline__ v8i b_operand(const uint8_t *frag, int q,
                                         uint32_t *bsc) {
  const int lane = threadIdx.x & 63, c = lane & 15, h = lane >> 4;
  const bool live = c < P;
  const int cc = live ? c : 0;
  const uint8_t *f = frag + frag_bytes(P) * q;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(f + 32 * (h * P + cc));
  const u32x4 b0 = src[0], b1 = src[1];
  *bsc = f[128 * P + h * P + cc];
  const uint32_t z = live ? 0xffffffffu : 0u;
  return v8i{(int)(b0.x & z), (int)(b0.y & z), (int)(b0.z & z), (int)(b0.w & z),
             (int)(b1.x & z), (int)(b1.y & z), (int)(b1.z & z), (int)(b1.w & z)};
}

// Inclusive prefix sum over the lanes of each 16-lane row, three steps: lane
// i < 8 ends with the sum of lanes 0..i of its row.
__device__ __forceinline__ float row_prefix8(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
  return v;
}

// Streams tiles [t_begin, t_end) of one matrix stack through the kNW waves
// of a workgroup, kMaxTPW tiles at a time. The chunk's (tile, quad) items
// are split into kNW contiguous runs, one per wave; a wave keeps four 16x16
// accumulators (one per 16-row sub-block of a quad), adds the P piece
// columns of each row when its run leaves a tile and stores the 64 row sums
// to its own LDS slot of that tile. The slots of a tile are then added in
// wave order, so every row has one summation order fixed by the shape.
//   base(t)  -> const uint8_t*  tile t's packed bytes (wave-uniform)
//   frag(t)  -> const uint8_t*  LDS fragments of the activation of tile t
//   pre()    -> ActPre          loads this wave's activations (runs first)
//   build(st)-> bool            builds the fragments from them (every wave
//                               takes part; runs once, after the first
//                               weight loads are in flight); true if an
//                               activation is not finite, and then nothing
//                               is computed
//   epi(t, lane, sum)           finished row sums of tile t, row = lane
// `part` is the caller's 16-byte aligned LDS array of kPartFloats floats.
// Returns false if build() reported a non-finite activation.
template <int P, class Base, class Frag, class Pre, class Build, class Epi>
__device__ __forceinline__ bool run_tiles_mfma(int t_begin, int t_end, int G4,
                                               Base base, Frag frag, Pre pre,
                                               Build build, Epi epi,
                                               float *part) {
  static_assert(P >= 1 && P <= 8, "row_prefix8 adds at most 8 columns");
  if (t_begin >= t_end) return true;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();

  // chunk state: tiles [c0, c0 + ntl), this wave's items [i0, i0 + nitems)
  int c0 = t_begin, ntl = 0, nitems = 0;
  int ltl = 0, lq = 0;  // next item to load (tile-local index, quad)
  const uint8_t *lbase = nullptr;  // base(c0 + ltl), refreshed per tile
  u32x4 a[kMfmaDepth][4];
  uint32_t asc[kMfmaDepth];
  auto setup = [&](int c) {
    c0 = c;
    ntl = min(kMaxTPW, t_end - c0);
    for (int tl = 0; tl < ntl; ++tl) part[(tl * kNW + wave) * 64 + lane] = 0.f;
    const int n = ntl * G4;
    const int i0 = wave * n / kNW;
    nitems = (wave + 1) * n / kNW - i0;
    ltl = i0 / G4;
    lq = i0 % G4;
    if (nitems > 0) lbase = base(c0 + ltl);
  };
  auto load = [&](int d) {
    const uint8_t *qb = lbase + (size_t)kQuadBytes * lq;
    const gu4_t *p = (const gu4_t *)(qb) + lane;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      a[d][m] = __builtin_nontemporal_load(p + (size_t)m * 64);
    asc[d] = __builtin_nontemporal_load((const gu32_t *)(qb + 4096) + lane);
    if (++lq == G4) {
      lq = 0;
      ++ltl;
      if (c0 + ltl < t_end) lbase = base(c0 + ltl);
    }
  };
  auto prologue = [&]() {
    if (nitems >= kMfmaDepth) {
#pragma unroll
      for (int d = 0; d < kMfmaDepth; ++d) load(d);
    } else {
#pragma unroll
      for (int d = 0; d < kMfmaDepth; ++d)
        if (d < nitems) load(d);
    }
  };

  // Consumes the chunk whose prologue is in flight, then writes its rows.
  auto stream_chunk = [&]() {
    int ktl = (wave * ntl * G4 / kNW) / G4, kq = (wave * ntl * G4 / kNW) % G4;
    int cur = ktl;  // tile the accumulators belong to
    const uint8_t *kfr = nitems > 0 ? frag(c0 + ktl) : nullptr;
    v4f acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
    auto flush = [&]() {
      // lane 16j + P-1 ends with rows 16m + 4j + i of tile `cur`
      v4f r[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) r[m][i] = row_prefix8(acc[m][i]);
      if ((lane & 15) == P - 1) {
        float *dst = part + (cur * kNW + wave) * 64 + 4 * (lane >> 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) *reinterpret_cast<v4f *>(dst + 16 * m) = r[m];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
    };
    auto consume = [&](int d) {
      if (ktl != cur) {
        flush();
        cur = ktl;
      }
      uint32_t bsc;
      const v8i bv = b_operand<P>(kfr, kq, &bsc);
      uint32_t e = asc[d];
      // groups with exponent byte 255 contribute nothing
      const uint32_t ff = (~e - 0x01010101u) & e & 0x80808080u;
      if (__ballot(ff != 0u)) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (((e >> (8 * m)) & 255u) == 255u) {
            a[d][m] = u32x4{0u, 0u, 0u, 0u};
            e &= ~(255u << (8 * m));
          }
      }
      // sub-block m takes byte m of the lane's exponent register (op_sel)
#define K3_MFMA_SUB(M)                                                         \
  {                                                                            \
    const u32x4 am = a[d][M];                                                  \
    const v8i av = {(int)am.x, (int)am.y, (int)am.z, (int)am.w, 0, 0, 0, 0};   \
    acc[M] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                 \
        av, bv, acc[M], 4, 0, M, (int)e, 0, (int)bsc);                         \
  }
      K3_MFMA_SUB(0)
      K3_MFMA_SUB(1)
      K3_MFMA_SUB(2)
      K3_MFMA_SUB(3)
#undef K3_MFMA_SUB
      if (++kq == G4) {
        kq = 0;
        ++ktl;
        if (c0 + ktl < t_end) kfr = frag(c0 + ktl);
      }
    };
    if (nitems >= kMfmaDepth) {
      int rem = nitems - kMfmaDepth;  // items not yet loaded
      for (; rem >= kMfmaDepth; rem -= kMfmaDepth) {
#pragma unroll
        for (int d = 0; d < kMfmaDepth; ++d) {
          consume(d);
          load(d);
        }
      }
#pragma unroll
      for (int d = 0; d < kMfmaDepth; ++d) {
        consume(d);
        if (d < rem) load(d);
      }
#pragma unroll
      for (int d = 0; d < kMfmaDepth; ++d)
        if (d < rem) consume(d);
    } else {
#pragma unroll
      for (int d = 0; d < kMfmaDepth; ++d)
        if (d < nitems) consume(d);
    }
    if (nitems > 0) flush();
    __syncthreads();
    for (int tl = wave; tl < ntl; tl += kNW) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) sum += part[(tl * kNW + w) * 64 + lane];
      epi(c0 + tl, lane, sum);
    }
    __syncthreads();
  };

  // Activation loads first, then the first chunk's weight loads, then the
  // fragments (waiting for the activations only), then the stream.
  {
    const ActPre st = pre();
    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads first
    setup(t_begin);
    prologue();
    __builtin_amdgcn_sched_barrier(0);
    if (__syncthreads_or(build(st) ? 1 : 0)) return false;
  }
  for (;;) {
    // Enter the loop with no load pending (the first consume needs these
    // bytes anyway): the loop's own waits then count only its own loads.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    stream_chunk();
    if (c0 + kMaxTPW >= t_end) break;
    setup(c0 + kMaxTPW);
    prologue();
  }
  return true;
}

// ---- VALU path for non-finite activations ------------------------------
// Same tiles and epilogue; each lane multiplies its own group with the
// E2M1 conversions and skips exponent-255 groups (group-then-scale), the
// four lanes of a row are added, and each slice's rows go to LDS.
//   dot(w, g, t) -> float   unscaled dot product of group g (lane-varying)
template <class Base, class Dot, class Epi>
__device__ __forceinline__ void run_tiles_valu(int t_begin, int t_end, int G,
                                               int G4, Base base, Dot dot,
                                               Epi epi, float *part) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  for (int c0 = t_begin; c0 < t_end; c0 += kMaxTPW) {
    const int ntl = min(kMaxTPW, t_end - c0);
    for (int tl = 0; tl < ntl; ++tl) {
      const int s = (wave + c0 + tl) % kNW;
      const uint8_t *tile = base(c0 + tl);
      float racc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int q = s * G4 / kNW; q < (s + 1) * G4 / kNW; ++q) {
        const uint8_t *qb = tile + (size_t)kQuadBytes * q;
        const uint32_t e = ((const uint32_t *)(qb + 4096))[lane];
        const int g = 4 * q + (lane >> 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32x4 w = ((const u32x4 *)(qb + 1024 * m))[lane];
          float d = 0.f;
          if (g < G) d = apply_scale(0.f, dot(w, g, c0 + tl), (e >> (8 * m)) & 255u);
          d += __shfl_xor(d, 16);
          d += __shfl_xor(d, 32);
          racc[m] += d;
        }
      }
      if (lane < 16) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          part[(tl * kNW + s) * 64 + 16 * m + lane] = racc[m];
      }
    }
    __syncthreads();
    for (int tl = wave; tl < ntl; tl += kNW) {
      float sum = 0.f;
#pragma unroll
      for (int s = 0; s < kNW; ++s) sum += part[(tl * kNW + s) * 64 + lane];
      epi(c0 + tl, lane, sum);
    }
    __syncthreads();
  }
}

}  // namespace k3
