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
constexpr int kPartFloats = kMaxTPW * kNW * 64;  // per-wave row partials, one vector

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left free (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// Streams tiles [t_begin, t_end) of one matrix stack with NA activation
// vectors per tile (NA = 1 for one token; the batched kernels multiply each
// decoded group by up to NA tokens), MaxTPW tiles per chunk.
//   base(t)               -> const uint8_t*  tile t's packed bytes (uniform)
//   na(t)                 -> int  vectors tile t uses (1..NA, uniform)
//   dot(w, g, t, n, sub)  sub[a] = unscaled dot of this lane's 16 code
//                            bytes w (group g of its row of tile t) with
//                            group g of activation vector a, for a < n =
//                            na(t) (g < G; g, t, n uniform)
//   epi(t, a, lane, s)    finished sum of row `lane` of tile t for vector a
//   pre()                 called once by every wave before any loaded quad
//                         is used: by waves 1.. after their first quads'
//                         loads are issued (a caller can wait there for its
//                         activations while the weights are on their way),
//                         by wave 0 before its own loads, since wave 0 is
//                         the one that polls and a poll completes only after
//                         the wave's earlier loads
// NWV waves per workgroup; `part` is the caller's LDS array of
// MaxTPW * NWV * 64 * NA floats.
struct NoPre {
  __device__ void operator()() const {}
};

template <int NA, int MaxTPW, int NWV = kNW, class Base, class Na, class Dot,
          class Epi, class Pre = NoPre>
__device__ __forceinline__ void run_rows_n(int t_begin, int t_end, int G,
                                           int G4, Base base, Na na, Dot dot,
                                           Epi epi, float *part,
                                           Pre pre = Pre()) {
  if (t_begin >= t_end) {
    pre();
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  auto slot = [&](int tl, int w, int a) { return ((tl * NWV + w) * NA + a) * 64; };

  // chunk state: tiles [c0, c0 + ntl), this wave's items [i0, i0 + nitems)
  int c0 = t_begin, ntl = 0, i0 = 0, nitems = 0;
  int ltl = 0, lq = 0;             // next item to load (tile-local, quad)
  const uint8_t *lbase = nullptr;  // base(c0 + ltl), refreshed per tile
  u32x4 a[kRingDepth][4];
  uint32_t asc[kRingDepth];
  auto setup = [&](int c) {
    c0 = c;
    ntl = min(MaxTPW, t_end - c0);
    for (int tl = 0; tl < ntl; ++tl)
#pragma unroll
      for (int v = 0; v < NA; ++v) part[slot(tl, wave, v) + lane] = 0.f;
    const int n = ntl * G4;
    i0 = wave * n / NWV;
    nitems = (wave + 1) * n / NWV - i0;
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
    int cur = ktl;                    // tile the accumulators belong to
    int cna = nitems > 0 ? na(c0 + ktl) : 0;
    float acc[NA];
#pragma unroll
    for (int v = 0; v < NA; ++v) acc[v] = 0.f;
    auto flush = [&]() {
#pragma unroll
      for (int v = 0; v < NA; ++v) {
        part[slot(cur, wave, v) + lane] = acc[v];
        acc[v] = 0.f;
      }
    };
    auto consume = [&](int d) {
      if (ktl != cur) {
        flush();
        cur = ktl;
        cna = na(c0 + ktl);
      }
      const uint32_t e = asc[d];
      const int g0 = 4 * kq;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (g0 + b < G) {
          const uint32_t eb = (e >> (8 * b)) & 255u;
          float sub[NA];
          dot(a[d][b], g0 + b, c0 + ktl, cna, sub);
#pragma unroll
          for (int v = 0; v < NA; ++v)
            if (v < cna) acc[v] = apply_scale(acc[v], sub[v], eb);
        }
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
    for (int tl = wave; tl < ntl; tl += NWV) {
      const int nv = na(c0 + tl);
#pragma unroll
      for (int v = 0; v < NA; ++v) {
        if (v >= nv) break;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) sum += part[slot(tl, w, v) + lane];
        epi(c0 + tl, v, lane, sum);
      }
    }
    __syncthreads();
  };

  setup(t_begin);
  for (bool first = true;; first = false) {
    if (first && wave == 0) pre();
    prologue();
    if (first && wave != 0) pre();
    // Enter the loop with no load pending (the first consume needs these
    // bytes anyway): the loop's own waits then count only its own loads.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    stream_chunk();
    if (c0 + MaxTPW >= t_end) break;
    setup(c0 + MaxTPW);
  }
}

// One activation vector per tile: the single-token kernels.
//   dot(w, g, t) -> float,  epi(t, lane, s)
template <class Base, class Dot, class Epi, class Pre = NoPre>
__device__ __forceinline__ void run_rows(int t_begin, int t_end, int G, int G4,
                                         Base base, Dot dot, Epi epi,
                                         float *part, Pre pre = Pre()) {
  run_rows_n<1, kMaxTPW>(
      t_begin, t_end, G, G4, base, [](int) { return 1; },
      [&](u32x4 w, int g, int t, int, float(&sub)[1]) { sub[0] = dot(w, g, t); },
      [&](int t, int, int lane, float s) { epi(t, lane, s); }, part, pre);
}

}  // namespace k3
