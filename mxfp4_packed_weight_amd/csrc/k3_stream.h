// Streaming loop of the single-token MXFP4 matrix-vector kernels.
//
// Every lane of a wave owns one row of a 64-row tile and every 16-byte lane
// load is one whole 32-code group of that row, so a wave's load of one group
// is a contiguous KiB. A quad (four groups of the 64 rows and their exponent
// bytes) is multiplied either on the matrix unit straight from those
// registers (k3_digits.h: four FP4 x FP8 instructions per quad against the
// activation vector's digits in LDS), or, when a workgroup's activations
// have a flagged group, group by group on the vector ALU (k3_decode.h), where
// the group's E8M0 exponent is applied once to the group's sum ([SAT]
// "Reduction one") and exponent byte 255 is skipped by a select ([A176] "What
// byte-identical actually costs"). Each route is its own instance of the
// loop, chosen once per workgroup, so the loop that runs holds one route.
//
// Work split: a workgroup owns a contiguous range of tiles and walks it
// kMaxTPW tiles at a time. The chunk's (tile, quad) items are cut into kNW
// contiguous runs, one per wave; a wave accumulates its row partial over the
// quads of its run, stores it to its LDS slot of that tile when the run
// leaves the tile, and the slots of a tile are added in wave order. Every row
// therefore has one summation order fixed by the shape, the grid and the
// route, and reruns are bit-identical ([SAT] "A floating-point contract, not
// a convention").
//
// Loads: a ring of kRingDepth quads per wave (four 16-byte code loads and
// one exponent dword per quad, non-temporal: each byte is read once). Every
// load in the steady loop is unconditional and the loop is entered with no
// load pending, so the compiler's wait counts are exact and the next quads
// stay in flight while one is multiplied.
#pragma once

#include "k3_decode.h"
#include "k3_digits.h"
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

// A workgroup barrier that orders LDS accesses only. __syncthreads() also
// waits for every global load the wave has in flight (vmcnt(0)), which would
// drain the quads of the ring issued just before it, and make every wave wait
// for the slowest wave's quads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Whether v holds in any thread of the workgroup, the same answer in every
// thread, through LDS behind lds_barrier(). (__syncthreads_or reads the
// workgroup size from the dispatch's argument block with vector loads and
// waits for them, and with them for every load in flight.) The flags are
// reused: two calls are separated by a barrier.
__device__ __forceinline__ bool wg_any(bool v) {
  __shared__ uint32_t any_flag[kNW];
  const bool w = __ballot(v) != 0ull;
  if ((threadIdx.x & 63) == 0) any_flag[wave_id()] = w ? 1u : 0u;
  lds_barrier();
  uint32_t a = 0u;
#pragma unroll
  for (int i = 0; i < kNW; ++i) a |= any_flag[i];
  return a != 0u;
}

struct NoPre {
  __device__ void operator()() const {}
};

// Streams tiles [t_begin, t_end) of one matrix stack, kMaxTPW tiles per
// chunk; kMx selects the route (true: matrix unit, false: vector ALU).
//   base(t)      -> const uint8_t*  tile t's packed bytes (uniform)
//   dig(t)       -> const lds_u8*   digits of tile t's activation vector
//                   (k3_digits.h, uniform; matrix route)
//   dot(w, g, t) -> float  unscaled dot of this lane's 16 code bytes w
//                   (group g of its row of tile t) with group g of tile t's
//                   activations (vector route; g, t uniform)
//   epi(t, lane, s)  finished sum of row `lane` of tile t
//   pre()        called once by every wave after its first quads' loads are
//                issued, before any is used: a caller can wait there for its
//                activations while the weights are on their way (a wave's
//                poll completes only after its earlier loads, which is no
//                loss: the quads are needed anyway)
//   fetch()      matrix route: called once by every wave right after pre(),
//                where activation loads that pre() waited for are issued
//   ready()      matrix route: called once by every wave after pre() and
//                after its first loads are issued, before any quad is used
//                (the workgroup builds its digits there; ends with a barrier)
//   ok()         matrix route: called once by every wave after ready();
//                false (the same in every wave) abandons the stream before
//                any quad is used, and run_rows returns false
// `part` is the caller's LDS array of kPartFloats floats. Returns true if the
// tiles were streamed.
template <bool kMx, class Base, class Dig, class Dot, class Epi, class Pre, class Fetch,
          class Ready, class Ok>
__device__ __forceinline__ bool run_rows(int t_begin, int t_end, int G, int G4, Base base,
                                         Dig dig, Dot dot, Epi epi, float *part, Pre pre,
                                         Fetch fetch, Ready ready, Ok ok) {
  if (t_begin >= t_end) {
    pre();
    if constexpr (kMx) {
      fetch();
      ready();
    }
    return true;
  }
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  auto slot = [&](int tl, int w) { return (tl * kNW + w) * 64; };

  // chunk state: tiles [c0, c0 + ntl), this wave's items [i0, i0 + nitems)
  int c0 = t_begin, ntl = 0, i0 = 0, nitems = 0;
  int ltl = 0, lq = 0;             // next item to load (tile-local, quad)
  const uint8_t *lbase = nullptr;  // base(c0 + ltl), refreshed per tile
  u32x4 a[kRingDepth][4];
  uint32_t asc[kRingDepth];
  auto setup = [&](int c) {
    c0 = c;
    ntl = min(kMaxTPW, t_end - c0);
    for (int tl = 0; tl < ntl; ++tl) part[slot(tl, wave) + lane] = 0.f;
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
    int cur = ktl;                    // tile the accumulators belong to
    // matrix route: block sums per 16-row block; vector route: the row sum
    f32x4 acc[4];
    float vacc = 0.f;
    const lds_u8 *D = nullptr;
    DigitLane dl{};
    if constexpr (kMx) {
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      dl = digit_lane();
      if (nitems > 0) D = dig(c0 + ktl);
    }
    auto flush = [&]() {
      if constexpr (kMx) {
        mx_flush(acc, part + slot(cur, wave));
      } else {
        part[slot(cur, wave) + lane] = vacc;
        vacc = 0.f;
      }
    };
    auto consume = [&](int d) {
      if (ktl != cur) {
        flush();
        cur = ktl;
        if constexpr (kMx) D = dig(c0 + ktl);
      }
      if constexpr (kMx) {
        mx_quad(a[d], asc[d], D, G4, kq, dl, acc);
      } else {
        const uint32_t e = asc[d];
        const int g0 = 4 * kq;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (g0 + b < G) vacc = apply_scale(vacc, dot(a[d][b], g0 + b, c0 + ktl), (e >> (8 * b)) & 255u);
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
    for (int tl = wave; tl < ntl; tl += kNW) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) sum += part[slot(tl, w) + lane];
      epi(c0 + tl, lane, sum);
    }
    __syncthreads();
  };

  setup(t_begin);
  for (bool first = true;; first = false) {
    prologue();
    if (first) {
      pre();
      if constexpr (kMx) fetch();
    }
    if constexpr (kMx) {
      if (first) {
        ready();
        if (!ok()) {  // the same in every wave: let the first loads land, give up
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          return false;
        }
      }
    }
    // Enter the loop with no load pending (the first consume needs these
    // bytes anyway): the loop's own waits then count only its own loads.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    stream_chunk();
    if (c0 + kMaxTPW >= t_end) break;
    setup(c0 + kMaxTPW);
  }
  return true;
}

// Whether a stack's tiles are long enough per workgroup for the matrix
// route: at least kMinMatrixQuads quads (the ceiling of tiles / grid,
// times G4). A shorter stream would spend longer building the activation
// digits than the matrix unit saves. The answer depends on the shape and
// the grid only, so a fused launch and the separate launches of the same
// stage (grid min(tiles, compute units) against compute units) agree.
constexpr int kMinMatrixQuads = 64;
__device__ __forceinline__ bool matrix_stream(int tiles, int G4) {
  const int per_wg = (tiles + (int)gridDim.x - 1) / (int)gridDim.x;
  return per_wg * G4 >= kMinMatrixQuads;
}

// One stack of tiles: on the matrix unit when `matrix` and ok() after
// ready(), else on the vector ALU (after a refusal pre() is called again;
// fetch(), ready() and ok() are not).
template <class Base, class Dig, class Dot, class Epi, class Pre, class Fetch, class Ready,
          class Ok>
__device__ __forceinline__ void stream_tiles(bool matrix, int t_begin, int t_end, int G, int G4,
                                             Base base, Dig dig, Dot dot, Epi epi, float *part,
                                             Pre pre, Fetch fetch, Ready ready, Ok ok) {
  if (!matrix ||
      !run_rows<true>(t_begin, t_end, G, G4, base, dig, dot, epi, part, pre, fetch, ready, ok))
    run_rows<false>(t_begin, t_end, G, G4, base, dig, dot, epi, part, pre, NoPre(), NoPre(),
                    []() { return true; });
}

}  // namespace k3
