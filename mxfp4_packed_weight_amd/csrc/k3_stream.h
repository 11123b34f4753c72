// Streaming loop of the MXFP4 matrix-vector kernels (vector ALU).
//
// Every lane of a wave owns one row of a 64-row tile and every 16-byte lane
// load is one whole 32-code group of that row, so a wave's load of one group
// is a contiguous KiB and all lanes need the same 32 activations: those are
// wave-uniform, live in scalar registers (the scalar cache broadcasts them to
// the workgroup's waves), and each VALU instruction takes them as an operand.
// A group's 32 codes are converted to floats in registers by gfx950's scaled
// FP4 conversions (the E2M1 table is in the hardware), multiplied by the
// activations with fp32 accumulation, and the group's E8M0 exponent is
// applied once to the group's sum ([SAT] "Reduction one"); exponent byte 255
// is skipped by a select ([A176] "What byte-identical actually costs").
//
// Work split: a workgroup owns a contiguous range of tiles and walks it
// kMaxTPW tiles at a time. The chunk's (tile, quad) items are cut into kNW
// contiguous runs, one per wave; a wave accumulates its row partial over the
// quads of its run, stores it to its LDS slot of that tile when the run
// leaves the tile, and the slots of a tile are added in wave order. Every row
// therefore has one summation order fixed by the shape and the grid, and
// reruns are bit-identical ([SAT] "A floating-point contract, not a
// convention").
//
// Loads: a ring of kRingDepth quads per wave (four 16-byte code loads and
// one exponent dword per quad, non-temporal: each byte is read once). Every
// load in the steady loop is unconditional and the loop is entered with no
// load pending, so the compiler's wait counts are exact and the next quads
// stay in flight while one is multiplied.
#pragma once

#include "k3_decode.h"
#include "k3_internal.h"

namespace k3 {

#ifndef K3_RING_DEPTH
#define K3_RING_DEPTH 2
#endif
constexpr int kRingDepth = K3_RING_DEPTH;
constexpr int kPartFloats = kMaxTPW * kNW * 64;  // per-wave row partials

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left free (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// Streams tiles [t_begin, t_end) of one matrix stack.
//   base(t)          -> const uint8_t*  tile t's packed bytes (wave-uniform)
//   dot(w, g, t)     -> float  unscaled dot of this lane's 16 code bytes w
//                               (group g of its row of tile t) with the
//                               activations of group g (g < G, uniform)
//   epi(t, lane, s)  finished sum of row `lane` of tile t
// `part` is the caller's LDS array of kPartFloats floats.
template <class Base, class Dot, class Epi>
__device__ __forceinline__ void run_rows(int t_begin, int t_end, int G, int G4,
                                         Base base, Dot dot, Epi epi,
                                         float *part) {
  if (t_begin >= t_end) return;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();

  // chunk state: tiles [c0, c0 + ntl), this wave's items [i0, i0 + nitems)
  int c0 = t_begin, ntl = 0, i0 = 0, nitems = 0;
  int ltl = 0, lq = 0;             // next item to load (tile-local, quad)
  const uint8_t *lbase = nullptr;  // base(c0 + ltl), refreshed per tile
  u32x4 a[kRingDepth][4];
  uint32_t asc[kRingDepth];
  auto setup = [&](int c) {
    c0 = c;
    ntl = min(kMaxTPW, t_end - c0);
    for (int tl = 0; tl < ntl; ++tl) part[(tl * kNW + wave) * 64 + lane] = 0.f;
    const int n = ntl * G4;
    i0 = wave * n / kNW;
    nitems = (wave + 1) * n / kNW - i0;
    ltl = i0 / G4;
    lq = i0 % G4;
    if (nitems > 0) lbase = base(c0 + ltl);
  };
  auto load = [&](int d) {
    const uint8_t *qb = lbase + (size_t)kQuadBytes * lq;
    const gu4_t *p = (const gu4_t *)(qb) + lane;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      a[d][b] = __builtin_nontemporal_load(p + (size_t)b * 64);
    asc[d] = __builtin_nontemporal_load((const gu32_t *)(qb + 4096) + lane);
    if (++lq == G4) {
      lq = 0;
      ++ltl;
      if (c0 + ltl < t_end) lbase = base(c0 + ltl);
    }
  };
  auto prologue = [&]() {
    if (nitems >= kRingDepth) {
#pragma unroll
      for (int d = 0; d < kRingDepth; ++d) load(d);
    } else {
#pragma unroll
      for (int d = 0; d < kRingDepth; ++d)
        if (d < nitems) load(d);
    }
  };

  // Consumes the chunk whose prologue is in flight, then hands out its rows.
  auto stream_chunk = [&]() {
    int ktl = i0 / G4, kq = i0 % G4;  // next item to consume
    int cur = ktl;                    // tile the accumulator belongs to
    float acc = 0.f;
    auto flush = [&]() {
      part[(cur * kNW + wave) * 64 + lane] = acc;
      acc = 0.f;
    };
    auto consume = [&](int d) {
      if (ktl != cur) {
        flush();
        cur = ktl;
      }
      const uint32_t e = asc[d];
      const int g0 = 4 * kq;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (g0 + b < G)
          acc = apply_scale(acc, dot(a[d][b], g0 + b, c0 + ktl), (e >> (8 * b)) & 255u);
      if (++kq == G4) {
        kq = 0;
        ++ktl;
      }
    };
    if (nitems >= kRingDepth) {
      int rem = nitems - kRingDepth;  // items not yet loaded
      for (; rem >= kRingDepth; rem -= kRingDepth) {
#pragma unroll
        for (int d = 0; d < kRingDepth; ++d) {
          consume(d);
          load(d);
        }
      }
#pragma unroll
      for (int d = 0; d < kRingDepth; ++d) {
        consume(d);
        if (d < rem) load(d);
      }
#pragma unroll
      for (int d = 0; d < kRingDepth; ++d)
        if (d < rem) consume(d);
    } else {
#pragma unroll
      for (int d = 0; d < kRingDepth; ++d)
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

  setup(t_begin);
  for (;;) {
    prologue();
    // Enter the loop with no load pending (the first consume needs these
    // bytes anyway): the loop's own waits then count only its own loads.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    stream_chunk();
    if (c0 + kMaxTPW >= t_end) break;
    setup(c0 + kMaxTPW);
  }
}

}  // namespace k3
