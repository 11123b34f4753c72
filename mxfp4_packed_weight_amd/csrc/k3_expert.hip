// MXFP4 matrix-vector kernels: plain GEMV, the routed expert's gate/up +
// SwiGLU stage, its down stage, the activation-fragment builder and the
// weighted combine.
//
// The matrix kernels are CU-persistent: the grid has one workgroup of kNW
// waves per compute unit, each workgroup owns a contiguous range of 64-row
// tiles (of one matrix, or of the k selected experts back to back) and
// streams it through the FP4 matrix unit (run_tiles_mfma, k3_mfma.h). Each
// row's sum has one fixed order that depends on the shape only, so reruns
// are bit-identical (the pages' rule that every row is summed by one owner
// in one order, [SAT] "A floating-point contract, not a convention"). The
// work is a memory-bound stream of packed bytes ("the wait is for bytes to
// arrive", [SAT] "Reduction one").
#include <atomic>

#include "k3_mfma.h"

namespace k3 {

namespace {

constexpr int kThreads = kNW * 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__global__ __launch_bounds__(kThreads) void gemv_f32_kernel(
    const float *__restrict__ x, const uint8_t *__restrict__ tiles, int rows,
    int cols, float *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xfrag[];
  __shared__ __attribute__((aligned(16))) float part[kPartFloats];
  const MatLayout m = mat_layout(rows, cols);
  int t0, t1;
  wg_range(m.ntiles, &t0, &t1);
  auto base = [&](int t) { return tiles + (size_t)t * m.tile_bytes; };
  auto epi = [&](int t, int lane, float s) {
    const int row = t * kTileRows + lane;
    if (row < rows) y[row] = s;
  };
  if (t0 >= t1) return;
  auto at = [&](int fb, int k) {
    const int i = 128 * fb + k;
    const float v = x[min(i, cols - 1)];
    return i < cols ? v : 0.f;
  };
  auto dst = [&](int fb) { return xfrag + frag_bytes(kPieces) * fb; };
  if (!run_tiles_mfma<kPieces>(
          t0, t1, m.G4, base, [&](int) { return (const uint8_t *)xfrag; },
          [&]() { return preload_acts(at, m.G4); },
          [&](const ActPre &st) { return build_frags<kPieces>(st, at, m.G4, dst); },
          epi, part))
    run_tiles_valu(
        t0, t1, m.G, m.G4, base,
        [&](u32x4 w, int g, int) { return group_dot_f32(w, x + (size_t)32 * g); },
        epi, part);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

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
  extern __shared__ __attribute__((aligned(16))) uint8_t xfrag[];
  __shared__ __attribute__((aligned(16))) float part[kPartFloats];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.gu.ntiles;
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  auto base = [&](int t) {
    return expert_base(experts, idx, single, t / T) +
           (size_t)(t % T) * L.gu.tile_bytes;
  };
  auto epi = [&](int t, int lane, float s) {
    const float u = __shfl_down(s, 32);  // lane l<32: gate row; l+32: up row
    int is_up, row;
    gu_lane_row(t % T, lane, &is_up, &row);
    if (lane < 32 && row < inter) h[(size_t)(t / T) * inter + row] = silu(s) * u;
  };
  if (t0 >= t1) return;
  auto at = [&](int fb, int k) {
    const int i = 128 * fb + k;
    const float v = bf16_to_f32(x[min(i, hidden - 1)]);
    return i < hidden ? v : 0.f;
  };
  auto dst = [&](int fb) { return xfrag + frag_bytes(kPieces) * fb; };
  if (!run_tiles_mfma<kPieces>(
          t0, t1, L.gu.G4, base, [&](int) { return (const uint8_t *)xfrag; },
          [&]() { return preload_acts(at, L.gu.G4); },
          [&](const ActPre &st) { return build_frags<kPieces>(st, at, L.gu.G4, dst); },
          epi, part)) {
    const uint32_t *xp = reinterpret_cast<const uint32_t *>(x);
    run_tiles_valu(
        t0, t1, L.gu.G, L.gu.G4, base,
        [&](u32x4 w, int g, int) { return group_dot_bf16(w, xp + (size_t)16 * g); },
        epi, part);
  }
}

// yp[j][r] = W_down(e_j)[r] . h[j], tiles of the k slots back to back. The
// fragments of h[j] for every slot j the workgroup's range touches are built
// in LDS (dynamic LDS of down_slots_spanned x ceil(inter/128) fragments).
__global__ __launch_bounds__(kThreads) void down_kernel(
    const float *__restrict__ h, const uint8_t *const *__restrict__ experts,
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ single,
    int nslots, int hidden, int inter, float *__restrict__ yp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t hfrag[];
  __shared__ __attribute__((aligned(16))) float part[kPartFloats];
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.down.ntiles;
  const int nkb = L.down.G4;
  const int slot_bytes = frag_bytes(kPieces) * nkb;
  int t0, t1;
  wg_range(nslots * T, &t0, &t1);
  if (t0 >= t1) return;
  const int j0 = t0 / T;
  auto base = [&](int t) {
    return expert_base(experts, idx, single, t / T) + L.down_offset +
           (size_t)(t % T) * L.down.tile_bytes;
  };
  auto frag = [&](int t) { return (const uint8_t *)hfrag + (t / T - j0) * slot_bytes; };
  auto epi = [&](int t, int ln, float s) {
    const int row = (t % T) * kTileRows + ln;
    if (row < hidden) yp[(size_t)(t / T) * hidden + row] = s;
  };
  const int nfb = ((t1 - 1) / T - j0 + 1) * nkb;  // blocks of every slot touched
  auto at = [&](int fb, int k) {
    const int i = 128 * (fb % nkb) + k;
    const float v = h[(size_t)(j0 + fb / nkb) * inter + min(i, inter - 1)];
    return i < inter ? v : 0.f;
  };
  auto dst = [&](int fb) { return hfrag + frag_bytes(kPieces) * fb; };
  if (!run_tiles_mfma<kPieces>(
          t0, t1, nkb, base, frag, [&]() { return preload_acts(at, nfb); },
          [&](const ActPre &st) { return build_frags<kPieces>(st, at, nfb, dst); },
          epi, part))
    run_tiles_valu(
        t0, t1, L.down.G, L.down.G4, base,
        [&](u32x4 w, int g, int t) {
          return group_dot_f32(w, h + (size_t)(t / T) * inter + (size_t)32 * g);
        },
        epi, part);
}

// y[i] = sum_j w[j] * yp[j][i] in rank order j = 0..k-1, then bf16 (RNE).
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ yp, const float *__restrict__ w, int k,
    int hidden, uint16_t *__restrict__ y, float *__restrict__ y_f32) {
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
  if (y_f32) y_f32[i] = acc;
  if (y) y[i] = f32_to_bf16_rne(acc);
}

unsigned grid_for_tiles(int total) {
  const int cus = num_cus();
  return (unsigned)(total < cus ? total : cus);
}

}  // namespace

size_t act_frag_bytes(int len) {
  return (size_t)((len + 127) / 128) * frag_bytes(kPieces);
}

int down_slots_spanned(int nslots, int hidden, int inter) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const int T = L.down.ntiles, total = nslots * T;
  const int grid = (int)grid_for_tiles(total);
  const int per_wg = (total + grid - 1) / grid;
  return min(nslots, (per_wg + T - 1) / T + 1);
}

namespace {
// Sets the kernel's dynamic LDS allowance once and refuses sizes beyond the
// device's LDS (minus the kernel's static arrays).
hipError_t lds_ok(const void *kernel, size_t dyn, size_t *limit_out) {
  static std::atomic<int> cap{0};
  int c = cap.load(std::memory_order_relaxed);
  if (c <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&c, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
            hipSuccess &&
        c > 0)
      cap.store(c, std::memory_order_relaxed);
    else
      c = 160 * 1024;  // gfx950's LDS per workgroup; not cached: no device answered
  }
  const size_t limit = (size_t)c - sizeof(float) * kPartFloats;
  if (limit_out) *limit_out = limit;
  if (dyn > limit) return hipErrorInvalidValue;
  if (dyn > 48 * 1024)
    return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)dyn);
  return hipSuccess;
}
}  // namespace

size_t max_dynamic_lds() {
  size_t limit = 0;
  (void)lds_ok(nullptr, 0, &limit);
  return limit;
}

hipError_t launch_gemv_f32(const float *x, const uint8_t *tiles, int rows,
                           int cols, float *y, hipStream_t s) {
  const MatLayout m = mat_layout(rows, cols);
  const size_t dyn = act_frag_bytes(cols);
  if (hipError_t e = lds_ok((const void *)gemv_f32_kernel, dyn, nullptr)) return e;
  hipLaunchKernelGGL(gemv_f32_kernel, dim3(grid_for_tiles(m.ntiles)),
                     dim3(kThreads), dyn, s, x, tiles, rows, cols, y);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t *x, const uint8_t *const *experts,
                          const int32_t *idx, const uint8_t *single,
                          int nslots, int hidden, int inter, float *h,
                          hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const size_t dyn = act_frag_bytes(hidden);
  if (hipError_t e = lds_ok((const void *)gate_up_kernel, dyn, nullptr)) return e;
  hipLaunchKernelGGL(gate_up_kernel,
                     dim3(grid_for_tiles(nslots * L.gu.ntiles)), dim3(kThreads),
                     dyn, s, x, experts, idx, single, nslots, hidden, inter, h);
  return hipGetLastError();
}

hipError_t launch_down(const float *h, const uint8_t *const *experts,
                       const int32_t *idx, const uint8_t *single, int nslots,
                       int hidden, int inter, float *yp, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const size_t dyn =
      (size_t)down_slots_spanned(nslots, hidden, inter) * act_frag_bytes(inter);
  if (hipError_t e = lds_ok((const void *)down_kernel, dyn, nullptr)) return e;
  hipLaunchKernelGGL(down_kernel,
                     dim3(grid_for_tiles(nslots * L.down.ntiles)),
                     dim3(kThreads), dyn, s, h, experts, idx, single, nslots,
                     hidden, inter, yp);
  return hipGetLastError();
}

hipError_t launch_combine(const float *yp, const float *w, int k, int hidden,
                          uint16_t *y, float *y_f32, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3((hidden + 255) / 256), dim3(256), 0,
                     s, yp, w, k, hidden, y, y_f32);
  return hipGetLastError();
}

}  // namespace k3
