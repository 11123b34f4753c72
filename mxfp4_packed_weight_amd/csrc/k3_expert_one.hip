// One routed expert (gate/up + SwiGLU, down) in one launch over every
// compute unit.
//
// A single expert is too little work for the decode layer's split: its 48
// gate/up tiles (7168/1536) would occupy 48 of the 256 compute units, and its
// two stages would each pay a launch. Here the gate/up tiles are cut along K
// into S chunks, one (tile, chunk) unit per workgroup, so the whole grid
// streams the gate/up bytes at once; every unit's row partials go to the
// workspace. Each workgroup that owns a down tile has issued the loads of its
// tile's first quads before the gate/up work, waits for every unit's
// arrival, sums the S partials of each gate and up row in chunk order, forms
// h = SiLU(g) * u in LDS and multiplies its down tile by it. One hand-off
// between workgroups, and the down bytes are on their way while it happens.
//
// Summation order, fixed by the shape and the grid: inside a unit, each wave
// sums its quads in order and the waves' sums are added in wave order; a
// row's units are added in chunk order; a down row's quads likewise. Reruns
// are bit-identical ([SAT] "A floating-point contract, not a convention").
// The group's exponent is applied after its 32-term sum, and exponent byte
// 255 skips the group ([SAT] "Reduction one"; [A176] "What byte-identical
// actually costs").
#include "k3_stream.h"
#include "k3_sync.h"

namespace k3 {

// Polls of the hand-off wait in this file's launch (per device; see
// set_expert_one_wait_limit).
__device__ int expert_one_wait_limit = kSpinLimit;

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = kNW * 64;

// sum_{i<32} E2M1(code_i) * h_i with h in LDS (32 values at hg, 16-byte
// aligned, the same for every lane: broadcast reads), in the order of
// group_dot_f32.
__device__ __forceinline__ float group_dot_lds(const u32x4 w, const float *hg) {
  const f32x4 *h4 = reinterpret_cast<const f32x4 *>(hg);
  float s = 0.f;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], 1.0f, 3);
    const f32x4 a = h4[2 * d], b = h4[2 * d + 1];
    s = fmaf(v0.x, a.x, s);
    s = fmaf(v0.y, a.y, s);
    s = fmaf(v1.x, a.z, s);
    s = fmaf(v1.y, a.w, s);
    s = fmaf(v2.x, b.x, s);
    s = fmaf(v2.y, b.y, s);
    s = fmaf(v3.x, b.z, s);
    s = fmaf(v3.y, b.w, s);
  }
  return s;
}

struct Quad {
  u32x4 w[4];
  uint32_t e;
};

// Quad q of a tile: this lane's four 16-byte groups and its exponent word.
__device__ __forceinline__ Quad load_quad(const uint8_t *tile, int q) {
  const int lane = threadIdx.x & 63;
  const uint8_t *qb = tile + (size_t)kQuadBytes * q;
  const gu4_t *p = (const gu4_t *)qb + lane;
  Quad Q;
#pragma unroll
  for (int b = 0; b < 4; ++b) Q.w[b] = __builtin_nontemporal_load(p + (size_t)b * 64);
  Q.e = __builtin_nontemporal_load((const gu32_t *)(qb + 4096) + lane);
  return Q;
}

// acc += the groups of quad q (groups past G are padding and skipped).
template <class Dot>
__device__ __forceinline__ float consume_quad(float acc, const Quad &Q, int q, int G, Dot dot) {
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (4 * q + b < G) acc = apply_scale(acc, dot(Q.w[b], 4 * q + b), (Q.e >> (8 * b)) & 255u);
  return acc;
}

// Row sums of the workgroup's waves, added in wave order by wave 0 and
// handed to out(lane, sum).
template <class Out>
__device__ __forceinline__ void wg_row_sum(float (*part)[64], float acc, Out out) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) s += part[w][lane];
    out(lane, s);
  }
  __syncthreads();
}

// P1[u][64]: row partials of gate/up unit u = tile * S + chunk (rows 0..31
// gate, 32..63 up). slots: one arrival word per workgroup, marked with val.
__global__ __launch_bounds__(kThreads) void expert_one_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ expert, int hidden,
    int inter, int S, float *__restrict__ y, float *__restrict__ h_out, float *P1,
    uint64_t *slots, uint64_t val) {
  __shared__ float part[kNW][64];
  __shared__ __attribute__((aligned(16))) float hl[K3_MAX_INTER];
  __shared__ int bad;
  const ExpertLayout L = expert_layout(hidden, inter);
  const int G = gridDim.x, b = blockIdx.x, wave = wave_id(), lane = threadIdx.x & 63;
  const int Tg = L.gu.ntiles, Td = L.down.ntiles, units = Tg * S;
  if (threadIdx.x == 0) bad = 0;

  // this workgroup's down tiles: d0 = G - 1 - b, then every G-th
  const int d0 = G - 1 - b, Gd = L.down.G, G4d = L.down.G4;
  const uint8_t *down = expert + L.down_offset;
  const bool pre = d0 < Td && wave < G4d;
  Quad first{};
  if (pre) first = load_quad(down + (size_t)d0 * L.down.tile_bytes, wave);

  // gate/up units b, b + G, ...: tile u / S, quads [c G4 / S, (c + 1) G4 / S)
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
  auto dot_x = [&](u32x4 w, int g) { return group_dot_bf16(w, xp + (size_t)16 * g); };
  const int G4 = L.gu.G4, Ggu = L.gu.G;
  for (int u = b; u < units; u += G) {
    const int t = u / S, c = u % S;
    const int qa = c * G4 / S, n = (c + 1) * G4 / S - qa;
    const int i0 = qa + wave * n / kNW, i1 = qa + (wave + 1) * n / kNW;
    const uint8_t *tile = expert + (size_t)t * L.gu.tile_bytes;
    float acc = 0.f;
    for (int q = i0; q < i1; q += 2) {  // two quads in flight
      const Quad A = load_quad(tile, q);
      Quad B{};
      if (q + 1 < i1) B = load_quad(tile, q + 1);
      acc = consume_quad(acc, A, q, Ggu, dot_x);
      if (q + 1 < i1) acc = consume_quad(acc, B, q + 1, Ggu, dot_x);
    }
    wg_row_sum(part, acc, [&](int ln, float s) { st_dev(P1 + (size_t)u * 64 + ln, s); });
  }
  arrive(slots, val);
  if (d0 >= Td) return;

  // every unit's partials are in: h = SiLU(g) * u into LDS. A thread takes
  // h values i and i + kThreads and issues the loads of both before adding
  // (in chunk order).
  if (wave == 0 && !wave_wait_range(slots, 0, min(units, G), val, expert_one_wait_limit) &&
      lane == 0)
    bad = 1;
  __syncthreads();
  const float *P = after_wait(P1);
  for (int i0 = threadIdx.x; i0 < inter; i0 += 2 * kThreads) {
    float g[2] = {0.f, 0.f}, up[2] = {0.f, 0.f};
    for (int c0 = 0; c0 < S; c0 += 4) {
      float vg[2][4], vu[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int i = min(i0 + m * kThreads, inter - 1);
        const float *pr = P + (size_t)(i / 32) * S * 64 + i % 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = min(c0 + j, S - 1);
          vg[m][j] = ld_dev(pr + (size_t)c * 64);
          vu[m][j] = ld_dev(pr + (size_t)c * 64 + 32);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c0 + j < S) {
            g[m] += vg[m][j];
            up[m] += vu[m][j];
          }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
      if (i0 + m * kThreads < inter) hl[i0 + m * kThreads] = silu(g[m]) * up[m];
  }
  __syncthreads();
  if (h_out && d0 == 0)
    for (int i = threadIdx.x; i < inter; i += kThreads) h_out[i] = hl[i];

  auto dot_h = [&](u32x4 w, int g) { return group_dot_lds(w, hl + 32 * g); };
  for (int d = d0; d < Td; d += G) {
    const uint8_t *tile = down + (size_t)d * L.down.tile_bytes;
    float acc = 0.f;
    for (int q = wave; q < G4d; q += kNW) {
      const Quad Q = (d == d0 && q == wave) ? first : load_quad(tile, q);
      acc = consume_quad(acc, Q, q, Gd, dot_h);
    }
    wg_row_sum(part, acc, [&](int ln, float s) {
      const int row = d * kTileRows + ln;
      if (row < hidden) y[row] = bad ? __builtin_nanf("") : s;
    });
  }
}

}  // namespace

hipError_t set_expert_one_wait_limit(int polls) {
  return hipMemcpyToSymbol(HIP_SYMBOL(expert_one_wait_limit), &polls, sizeof(polls));
}

int expert_one_split(int hidden, int inter) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const int G = (int)moe_experts_grid();
  int S = G / L.gu.ntiles;
  if (S > L.gu.G4) S = L.gu.G4;
  return S < 1 ? 1 : S;
}

size_t expert_one_workspace_bytes(int hidden, int inter) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const int units = L.gu.ntiles > kMaxSyncGrid ? L.gu.ntiles : kMaxSyncGrid;
  return (((size_t)units * 64 * sizeof(float) + 255) & ~(size_t)255) +
         (size_t)kMaxSyncGrid * sizeof(uint64_t);
}

hipError_t launch_expert_one(const uint16_t *x, const uint8_t *expert, int hidden, int inter,
                             float *y, float *h, void *ws, uint64_t val, hipStream_t s) {
  const int S = expert_one_split(hidden, inter);
  const ExpertLayout L = expert_layout(hidden, inter);
  const int units = L.gu.ntiles > kMaxSyncGrid ? L.gu.ntiles : kMaxSyncGrid;
  float *P1 = static_cast<float *>(ws);
  uint64_t *slots = reinterpret_cast<uint64_t *>(
      static_cast<uint8_t *>(ws) + (((size_t)units * 64 * sizeof(float) + 255) & ~(size_t)255));
  return grid_sync_launch(s, [&]() {
    hipLaunchKernelGGL(expert_one_kernel, dim3(moe_experts_grid()), dim3(kThreads), 0, s, x,
                       expert, hidden, inter, S, y, h, P1, slots, val);
    return hipGetLastError();
  });
}

}  // namespace k3
