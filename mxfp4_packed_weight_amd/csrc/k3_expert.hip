// MXFP4 matrix-vector kernels: plain GEMV, the routed expert's gate/up +
// SwiGLU stage, its down stage and the weighted combine.
//
// The matrix kernels are CU-persistent: the grid has one workgroup of kNW
// waves per compute unit, each workgroup owns a contiguous range of 64-row
// tiles (of one matrix, or of the k selected experts back to back) and
// streams it through run_rows (k3_stream.h), which multiplies the packed
// codes on the matrix unit against the activations' digits, built by the
// workgroup in LDS while its first loads are in flight (k3_digits.h). Each row's sum has one fixed order that depends on the shape and grid
// only, so reruns are bit-identical (the pages' rule that every row is summed
// by one owner in one order, [SAT] "A floating-point contract, not a
// convention"). The work is a memory-bound stream of packed bytes ("the wait
// is for bytes to arrive", [SAT] "Reduction one").
#include <functional>
#include <mutex>

#include "k3_stream.h"
#include "k3_shared_row.h"
#include "k3_sync.h"
#include "k3_topk.h"

namespace k3 {

// Polls of each hand-off wait in this file's launches (per device; see
// set_expert_wait_limit).
__device__ int expert_wait_limit = kSpinLimit;

namespace {

constexpr int kThreads = kNW * 64;

// LDS digits of the activation vectors of slots [s_lo, s_hi], as many as
// fit (n); `all` if every slot fits.
struct SlotDigits {
  lds_u8 *buf;
  int s_lo, n, stride;
  bool all;
  __device__ const lds_u8 *at(int s) const { return buf + (s - s_lo) * stride; }
};

// The slots of tiles [t0, t1) of a stack of T tiles per slot.
__device__ __forceinline__ SlotDigits slot_digits(uint8_t *buf, int t0, int t1, int T, int G4) {
  SlotDigits d;
  d.buf = (lds_u8 *)buf;
  d.stride = digit_bytes(G4);
  d.s_lo = t0 / T;
  const int want = t0 < t1 ? (t1 - 1) / T - d.s_lo + 1 : 0;
  d.n = min(want, kDigitLds / d.stride);
  d.all = d.n == want;
  return d;
}

// Builds every slot's digits (load(s, i) = element i of slot s's vector) and
// returns, the same in every thread, whether the matrix route may run: every
// slot fits and no group is flagged.
template <class Load>
__device__ __forceinline__ bool build_slot_digits(const SlotDigits &d, int G, int G4, Load load) {
  bool flagged = false;
  for (int i = 0; i < d.n; ++i)
    flagged |= build_digits([&](int k) { return load(d.s_lo + i, k); }, G, G4, d.buf + i * d.stride);
  return !wg_any(flagged) && d.all;
}

// The bf16 activation vector x (hidden values) of the gate/up stages: its
// bytes go to LDS behind the digits by direct copies when both fit (true),
// for the digits to be computed there later.
__device__ __forceinline__ bool stage_x(const uint16_t *x, int hidden, const SlotDigits &d) {
  const int at = d.stride, bytes = 2 * hidden;
  if (d.n < 1 || at + bytes > kDigitLds) return false;
  dma_to_lds(reinterpret_cast<const uint8_t *>(x), d.buf + at, bytes);
  return true;
}

// x's digits into D's one vector (from the LDS copy when staged, else from
// device memory); whether the matrix route may run (as build_slot_digits).
__device__ __forceinline__ bool x_ready(const uint16_t *x, bool staged, int G, int G4,
                                        const SlotDigits &d) {
  if (staged) {
    const bool flagged = compute_digits_bf16(d.buf + d.stride, G, G4, d.buf);
    return !wg_any(flagged) && d.all;
  }
  return build_slot_digits(d, G, G4,
                           [&](int, int i) { return __uint_as_float((uint32_t)x[i] << 16); });
}

__global__ __launch_bounds__(kThreads) void gemv_f32_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ tiles, int rows,
    int cols, float *__restrict__ y) {
  __shared__ float part[kPartFloats];
  __shared__ __attribute__((aligned(16))) uint8_t dig[kDigitLds];
  const MatLayout m = mat_layout(rows, cols);
  int t0, t1;
  wg_range(m.ntiles, &t0, &t1);
  // one vector for every tile (wider than the buffer: the vector-ALU route)
  const SlotDigits D = slot_digits(dig, 0, 1, 1, m.G4);
  bool mx = false;
  stream_tiles(
      matrix_stream(m.ntiles, m.G4), t0, t1, m.G, m.G4,
      [&](int t) { return tiles + (size_t)t * m.tile_bytes; },
      [&](int) { return D.at(0); },
      [&](u32x4 w, int g, int) { return group_dot_f32(w, x + (size_t)32 * g); },
      [&](int t, int lane, float s) {
        const int row = t * kTileRows + lane;
        if (row < rows) y[row] = s;
      },
      part, NoPre(), NoPre(),
      [&]() { mx = build_slot_digits(D, m.G, m.G4, [&](int, int i) { return x[i]; }); },
      [&]() { return mx; });
}

__device__ __forceinline__ const uint8_t *expert_base(
    const uint8_t *const *__restrict__ experts, const int32_t *__restrict__ idx,
    const uint8_t *single, int slot) {
  return experts ? experts[idx[slot]] : single;
}

// Tiles of the k slots back to back: tile t is gate/up tile t % T of slot
// t / T (T tiles per expert). h[j][i] = SiLU(gate_i . x) * (up_i . x).
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t *__restrict__ x, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ h) {
  __shared__ float part[kPartFloats];
  __shared__ __attribute__((aligned(16))) uint8_t dig[kDigitLds];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.gu.ntiles;
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  const SlotDigits D = slot_digits(dig, 0, 1, 1, L.gu.G4);  // x, shared by every slot
  bool mx = false;
  stream_tiles(
      matrix_stream(nslots * T, L.gu.G4), t0, t1, L.gu.G, L.gu.G4,
      [&](int t) {
        return expert_base(experts, idx, single, t / T) +
               (size_t)(t % T) * L.gu.tile_bytes;
      },
      [&](int) { return D.at(0); },
      [&](u32x4 w, int g, int) { return group_dot_bf16(w, xp + (size_t)16 * g); },
      [&](int t, int lane, float s) {
        const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
        int is_up, row;
        gu_lane_row(t % T, lane, &is_up, &row);
        if (lane < 32 && row < inter) h[(size_t)(t / T) * inter + row] = silu(s) * u;
      },
      part, NoPre(), NoPre(), [&]() { mx = x_ready(x, false, L.gu.G, L.gu.G4, D); },
      [&]() { return mx; });
}

// yp[j][r] = W_down(e_j)[r] . h[j], tiles of the k slots back to back (a
// workgroup's tiles share one or two slots, so its activations stay within
// the scalar cache).
__global__ __launch_bounds__(kThreads) void down_kernel(
    const float *__restrict__ h, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ yp) {
  __shared__ float part[kPartFloats];
  __shared__ __attribute__((aligned(16))) uint8_t dig[kDigitLds];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.down.ntiles;
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  const SlotDigits D = slot_digits(dig, t0, t1, T, L.down.G4);
  bool mx = false;
  stream_tiles(
      matrix_stream(nslots * T, L.down.G4), t0, t1, L.down.G, L.down.G4,
      [&](int t) {
        return expert_base(experts, idx, single, t / T) + L.down_offset +
               (size_t)(t % T) * L.down.tile_bytes;
      },
      [&](int t) { return D.at(t / T); },
      [&](u32x4 w, int g, int t) {
        return group_dot_f32(w, h + (size_t)(t / T) * inter + (size_t)32 * g);
      },
      [&](int t, int lane, float s) {
        const int row = (t % T) * kTileRows + lane;
        if (row < hidden) yp[(size_t)(t / T) * hidden + row] = s;
      },
      part, NoPre(), NoPre(),
      [&]() {
        mx = build_slot_digits(D, L.down.G, L.down.G4,
                               [&](int sl, int i) { return h[(size_t)sl * inter + i]; });
      },
      [&]() { return mx; });
}

// The decode layer's first expert stage with the selection folded in:
// every workgroup ranks the token's n logits itself with all of its waves
// (topk_wg: the same selection everywhere, so no grid-wide step is needed),
// workgroup 0 publishes idx and w, then the tiles of the k selected
// experts' gate/up stacks are streamed as in gate_up_kernel. One launch
// fewer than a separate top-k.
__global__ __launch_bounds__(kThreads) void gate_up_routed_kernel(
    const uint16_t *__restrict__ x, const double *__restrict__ logits,
    const uint8_t *const *__restrict__ experts, int n, int k, int hidden,
    int inter, float *__restrict__ h, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out) {
  __shared__ float part[kPartFloats];
  __shared__ __attribute__((aligned(16))) uint8_t dig[kDigitLds];
  __shared__ TopkWgLds tk;
  const ExpertLayout L = expert_layout(hidden, inter);
  const SlotDigits D = slot_digits(dig, 0, 1, 1, L.gu.G4);
  // x's bytes on their way to LDS, when the gate/up tiles take the matrix route
  const bool staged = matrix_stream(k * L.gu.ntiles, L.gu.G4) && stage_x(x, hidden, D);
  topk_wg<kNW>(logits, n, k, tk);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's copies are in
  __syncthreads();
  if (blockIdx.x == 0 && (int)threadIdx.x < k) {
    idx_out[threadIdx.x] = tk.sel[threadIdx.x];
    w_out[threadIdx.x] = tk.wt[threadIdx.x];
  }
  const int T = L.gu.ntiles;
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
  int t0, t1;
  wg_range(k * T, &t0, &t1);
  bool mx = false;
  stream_tiles(
      matrix_stream(k * T, L.gu.G4), t0, t1, L.gu.G, L.gu.G4,
      [&](int t) {
        const int e = __builtin_amdgcn_readfirstlane(tk.sel[t / T]);
        return ldc(experts + e) + (size_t)(t % T) * L.gu.tile_bytes;
      },
      [&](int) { return D.at(0); },
      [&](u32x4 w, int g, int) { return group_dot_bf16(w, xp + (size_t)16 * g); },
      [&](int t, int lane, float s) {
        const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
        int is_up, row;
        gu_lane_row(t % T, lane, &is_up, &row);
        if (lane < 32 && row < inter) h[(size_t)(t / T) * inter + row] = silu(s) * u;
      },
      part, NoPre(), NoPre(), [&]() { mx = x_ready(x, staged, L.gu.G, L.gu.G4, D); },
      [&]() { return mx; });
}

// The decode layer's expert work in one launch, after the router: top-k
// (topk_wg), gate/up + SwiGLU, down, and the weighted combine. The grid is
// one workgroup per compute unit; each stage cuts its tiles over the grid as
// the separate kernels do (gate_up_routed_kernel, down_kernel, then
// combine_kernel), so the bits equal those launches'. Between stages:
//   - h goes out with device-coherent stores and each workgroup marks its
//     stage-0 arrival slot with the call's value `val`; a workgroup's down
//     stage issues its first quads' loads and then waits only for the
//     workgroups that produced the h slots it needs (its own expert's
//     gate/up workgroups), so the down weights are already on their way;
//   - the down partials go out the same way (stage-1 slots); the owner of a
//     row tile's last partial waits for the owners of the others and sums
//     the k partials in rank order.
// This saves the boundary between the gate/up and down launches, the down
// launch's ramp and the combine launch. Waits are bounded: if the device
// cannot run the whole grid at once for about a second (another kernel
// holding compute units), the call writes NaN rather than hang.
//
// kShared: the layer also has shared experts, whose h (hs) an earlier launch
// computed. Between its gate/up and down stages every workgroup takes its
// slice of the shared down rows (shared_down_row, the bits of the separate
// shared-down launch), while its expert's h may still be on its way; their
// sums ys go out device-coherent, and the combine adds them after the routed
// rank-order sum. Without kShared, `add` (optional) is a finished vector
// from an earlier launch.
template <bool kShared>
__global__ __launch_bounds__(kThreads) void moe_experts_kernel(
    const uint16_t *__restrict__ x, const double *__restrict__ logits,
    const uint8_t *const *__restrict__ experts, int n, int k, int hidden,
    int inter, float *h, float *yp, uint64_t *slots, uint64_t val,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    uint16_t *__restrict__ y, float *__restrict__ y_f32,
    const float *add, const float *__restrict__ hs,
    const uint16_t *const *__restrict__ shared, int n_shared, int inter_s) {
  __shared__ float part[kPartFloats];
  __shared__ __attribute__((aligned(16))) uint8_t dig[kDigitLds];  // x's, then h's
  __shared__ TopkWgLds tk;
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  const ExpertLayout L = expert_layout(hidden, inter);
  const SlotDigits D = slot_digits(dig, 0, 1, 1, L.gu.G4);
  // x's bytes on their way to LDS, when the gate/up tiles take the matrix route
  const bool staged = matrix_stream(k * L.gu.ntiles, L.gu.G4) && stage_x(x, hidden, D);
  topk_wg<kNW, false>(logits, n, k, tk);  // the weights come during the wait for h
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's copies are in
  __syncthreads();
  const int G = gridDim.x, lane = threadIdx.x & 63;
  const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
  const int Tg = L.gu.ntiles, total_gu = k * Tg;
  {
    int t0, t1;
    wg_range(total_gu, &t0, &t1);
    bool mx = false;
    stream_tiles(
        matrix_stream(total_gu, L.gu.G4), t0, t1, L.gu.G, L.gu.G4,
        [&](int t) {
          const int e = __builtin_amdgcn_readfirstlane(tk.sel[t / Tg]);
          return ldc(experts + e) + (size_t)(t % Tg) * L.gu.tile_bytes;
        },
        [&](int) { return D.at(0); },
        [&](u32x4 w, int g, int) { return group_dot_bf16(w, xp + (size_t)16 * g); },
        [&](int t, int ln, float s) {
          const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
          int is_up, row;
          gu_lane_row(t % Tg, ln, &is_up, &row);
          if (ln < 32 && row < inter)
            st_dev(h + (size_t)(t / Tg) * inter + row, silu(s) * u);
        },
        part, NoPre(), NoPre(), [&]() { mx = x_ready(x, staged, L.gu.G, L.gu.G4, D); },
        [&]() { return mx; });
  }
  arrive(slots, val);
  if constexpr (kShared) {
    int r0, r1;
    wg_range(hidden, &r0, &r1);
    for (int r = r0 + wave_id(); r < r1; r += kNW) {
      const float v = shared_down_row(hs, shared, n_shared, hidden, inter_s, r);
      if (lane == 0) st_dev(const_cast<float *>(add) + r, v);
    }
  }

  const int Td = L.down.ntiles, total = k * Td;
  int t0, t1;
  wg_range(total, &t0, &t1);
  const float *hb = h;
  const SlotDigits Dd = slot_digits(dig, t0, t1, Td, L.down.G4);
  bool mxd = false;
  stream_tiles(
      matrix_stream(total, L.down.G4), t0, t1, L.down.G, L.down.G4,
      [&](int t) {
        const int e = __builtin_amdgcn_readfirstlane(tk.sel[t / Td]);
        return ldc(experts + e) + L.down_offset + (size_t)(t % Td) * L.down.tile_bytes;
      },
      [&](int t) { return Dd.at(t / Td); },
      [&](u32x4 w, int g, int t) {
        return group_dot_f32(w, hb + (size_t)(t / Td) * inter + (size_t)32 * g);
      },
      [&](int t, int ln, float s) {
        const int row = (t % Td) * kTileRows + ln;
        if (row < hidden) st_dev(yp + (size_t)(t / Td) * hidden + row, s);
      },
      part,
      [&]() {  // the gate/up workgroups of this workgroup's down slots
        if (t0 < t1 && wave_id() == 0) {
          const int c_lo = tile_owner(t0 / Td * Tg, total_gu, G);
          const int c_hi = tile_owner(((t1 - 1) / Td + 1) * Tg - 1, total_gu, G);
          if (!wave_wait_range(slots, c_lo, c_hi - c_lo + 1, val, expert_wait_limit) &&
              lane == 0)
            bad = 1;
        }
        lds_barrier();  // wave 0's poll has returned; the quads stay in flight
        hb = after_wait(hb);
      },
      NoPre(),
      [&]() {  // h of this workgroup's slots, device-coherent, into digits
        mxd = build_slot_digits(Dd, L.down.G, L.down.G4,
                                [&](int sl, int i) { return ld_dev(hb + (size_t)sl * inter + i); });
      },
      [&]() { return mxd; });
  uint64_t *done = slots + kMaxSyncGrid;
  arrive(done, val);

  const int last = (k - 1) * Td;
  const int r_lo = max(t0 - last, 0), r_hi = min(t1 - last, Td);
  // The routing weights (lane j < k: rank j's), in the registers of each wave
  // that needs them: here they are off the path to the experts' loads, and
  // a combining wave usually waits for other workgroups' partials anyway.
  const bool publish = blockIdx.x == 0 && wave_id() == kNW - 1;
  const float wl = r_lo + wave_id() < r_hi || publish ? topk_wg_weight_lane(tk, k) : 0.f;
  if (publish && lane < k) {
    idx_out[lane] = tk.sel[lane];
    w_out[lane] = wl;
  }
  for (int r = r_lo + wave_id(); r < r_hi; r += kNW) {
    const int owner = lane < k ? tile_owner(lane * Td + r, total, G) : 0;
    if (!wave_wait_owners(done, owner, k, val, expert_wait_limit) && lane == 0) bad = 1;
    if constexpr (kShared) {  // the workgroups that wrote these rows of ys
      const int s_lo = tile_owner(r * kTileRows, hidden, G);
      const int s_hi = tile_owner(min((r + 1) * kTileRows, hidden) - 1, hidden, G);
      if (!wave_wait_range(done, s_lo, s_hi - s_lo + 1, val, expert_wait_limit) && lane == 0)
        bad = 1;
    }
    const int row = r * kTileRows + lane;
    if (row < hidden) {
      float acc = 0.f;
      for (int j0 = 0; j0 < k; j0 += 16) {  // as combine_kernel
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          v[j] = j0 + j < k ? ld_dev(yp + (size_t)(j0 + j) * hidden + row) : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j0 + j < k)
            acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j0 + j)),
                       v[j], acc);
      }
      if (kShared)
        acc += ld_dev(add + row);  // the shared experts' output, from this launch
      else if (add)
        acc += add[row];
      if (y_f32) y_f32[row] = acc;
      if (y) y[row] = f32_to_bf16_rne(acc);
    }
  }
  __syncthreads();
  if (bad)  // the outputs cannot be trusted: say so in them
    for (int i = threadIdx.x; i < hidden; i += kThreads) {
      if (y_f32) y_f32[i] = __builtin_nanf("");
      if (y) y[i] = 0x7FC0;
    }
}

// y[i] = sum_j w[j] * yp[j][i] in rank order j = 0..k-1 (+ add[i] when
// given), then bf16 (RNE).
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ yp, const float *__restrict__ w, int k,
    int hidden, uint16_t *__restrict__ y, float *__restrict__ y_f32,
    const float *__restrict__ add) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= hidden) return;
  float acc = 0.f;
  for (int j0 = 0; j0 < k; j0 += 16) {  // issue a batch of loads, then add
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = j0 + j < k ? yp[(size_t)(j0 + j) * hidden + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j0 + j < k) acc = fmaf(w[j0 + j], v[j], acc);
  }
  if (add) acc += add[i];
  if (y_f32) y_f32[i] = acc;
  if (y) y[i] = f32_to_bf16_rne(acc);
}

#ifndef K3_WG_PER_CU
#define K3_WG_PER_CU 1
#endif
unsigned grid_for_tiles(int total) {
  const int wgs = num_cus() * K3_WG_PER_CU;
  return (unsigned)(total < wgs ? total : wgs);
}

}  // namespace

hipError_t launch_gemv_f32(const float *x, const uint8_t *tiles, int rows,
                           int cols, float *y, hipStream_t s) {
  const MatLayout m = mat_layout(rows, cols);
  hipLaunchKernelGGL(gemv_f32_kernel, dim3(grid_for_tiles(m.ntiles)),
                     dim3(kThreads), 0, s, x, tiles, rows, cols, y);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t *x, const uint8_t *const *experts,
                          const int32_t *idx, const uint8_t *single,
                          int nslots, int hidden, int inter, float *h,
                          hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(gate_up_kernel,
                     dim3(grid_for_tiles(nslots * L.gu.ntiles)), dim3(kThreads),
                     0, s, x, experts, idx, single, nslots, hidden, inter, h);
  return hipGetLastError();
}

hipError_t launch_down(const float *h, const uint8_t *const *experts,
                       const int32_t *idx, const uint8_t *single, int nslots,
                       int hidden, int inter, float *yp, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(down_kernel,
                     dim3(grid_for_tiles(nslots * L.down.ntiles)),
                     dim3(kThreads), 0, s, h, experts, idx, single, nslots,
                     hidden, inter, yp);
  return hipGetLastError();
}

hipError_t launch_gate_up_routed(const uint16_t *x, const double *logits,
                                 const uint8_t *const *experts, int n, int k,
                                 int hidden, int inter, float *h, int32_t *idx,
                                 float *w, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  hipLaunchKernelGGL(gate_up_routed_kernel, dim3(grid_for_tiles(k * L.gu.ntiles)),
                     dim3(kThreads), 0, s, x, logits, experts, n, k, hidden,
                     inter, h, idx, w);
  return hipGetLastError();
}

unsigned moe_experts_grid() { return (unsigned)num_cus(); }

hipError_t set_expert_wait_limit(int polls) {
  return hipMemcpyToSymbol(HIP_SYMBOL(expert_wait_limit), &polls, sizeof(polls));
}

namespace {
// Two launches whose workgroups wait for each other (this file's expert
// launch, the one-expert launch) must never run at the same time on one
// device: each needs all of its workgroups resident, and two grids that each
// hold part of the compute units would both wait until their polls run out.
// Calls on one stream are ordered by the stream. While every such launch on
// a device has gone to one stream nothing more is done (an event per launch
// costs a few microseconds of the layer). The first launch on a second
// stream waits on the host until the device is idle, so the previous
// stream's launches are finished without touching that stream (it may no
// longer exist); from then on an event is recorded after every launch, and a
// launch on another stream than the previous one waits for it on the device.
struct FusedOrder {
  std::mutex mu;
  hipStream_t last = nullptr;
  hipEvent_t done = nullptr;
  bool any = false;    // a launch went out on this device
  bool multi = false;  // launches went to more than one stream
};
FusedOrder g_fused_order[kMaxDevices];
}  // namespace

hipError_t grid_sync_launch(hipStream_t s, const std::function<hipError_t()> &launch) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  FusedOrder &o = g_fused_order[dev];
  std::lock_guard<std::mutex> lock(o.mu);
  if (o.any && o.last != s) {
    if (!o.multi) {  // first switch of stream: finish everything queued so far
      hipError_t e = hipEventCreateWithFlags(&o.done, hipEventDisableTiming);
      if (e != hipSuccess) {
        o.done = nullptr;
        return e;
      }
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return e;
      o.multi = true;
    } else {
      const hipError_t e = hipStreamWaitEvent(s, o.done, 0);
      if (e != hipSuccess) return e;
    }
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (o.multi) {
    e = hipEventRecord(o.done, s);
    if (e != hipSuccess) return e;
  }
  o.last = s;
  o.any = true;
  return hipSuccess;
}

hipError_t launch_moe_experts(const uint16_t *x, const double *logits,
                              const uint8_t *const *experts, int n, int k,
                              int hidden, int inter, float *h, float *yp,
                              uint64_t *slots, uint64_t val, int32_t *idx,
                              float *w, uint16_t *y, float *y_f32,
                              hipStream_t s, const float *add, const SharedStage *sh) {
  // one workgroup per compute unit: the whole grid fits at once
  return grid_sync_launch(s, [&]() {
    if (sh)
      hipLaunchKernelGGL(moe_experts_kernel<true>, dim3(moe_experts_grid()), dim3(kThreads), 0,
                         s, x, logits, experts, n, k, hidden, inter, h, yp, slots, val, idx, w,
                         y, y_f32, sh->ys, sh->hs, sh->shared, sh->n_shared, sh->inter);
    else
      hipLaunchKernelGGL(moe_experts_kernel<false>, dim3(moe_experts_grid()), dim3(kThreads), 0,
                         s, x, logits, experts, n, k, hidden, inter, h, yp, slots, val, idx, w,
                         y, y_f32, add, nullptr, nullptr, 0, 0);
    return hipGetLastError();
  });
}

hipError_t launch_combine(const float *yp, const float *w, int k, int hidden,
                          uint16_t *y, float *y_f32, hipStream_t s, const float *add) {
  hipLaunchKernelGGL(combine_kernel, dim3((hidden + 255) / 256), dim3(256), 0,
                     s, yp, w, k, hidden, y, y_f32, add);
  return hipGetLastError();
}

}  // namespace k3
