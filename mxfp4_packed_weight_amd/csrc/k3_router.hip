// Router: bf16 logits GEMV in fp64 and sigmoid top-k selection.
//
// Logits: one wave per (token, expert) row. Each lane issues the loads of
// all its 16-byte chunks of the bf16 router row (and of x) before computing,
// so the whole router matrix is in flight at once; products are formed in
// fp64 (a product of two bf16 values is exact there) into four chains per
// lane, and the lane sums are combined by a fixed DPP tree, so the logits
// are reproducible bit for
// bit and within ~1e-16 of a sequential fp64 sum, which keeps the top-k
// indices identical to an fp64 reference.
//
// Selection: one wave per token with the keys in registers; a cheap lower
// bound keeps ~18 candidates, which are ranked in parallel (see
// topk_kernel). Ties go to the lower expert index. The routing bias only
// changes the keys; the weights always come from the unbiased sigmoid scores
// ([ZOR] "How is the C engine actually built?", invariant 3), renormalised to
// sum to one, summed in rank order.
#include <limits.h>
#include <math.h>

#include "k3_decode.h"
#include "k3_internal.h"

namespace k3 {

namespace {

__device__ __forceinline__ double bf16_lo(uint32_t v) {
  return (double)__uint_as_float(v << 16);
}
__device__ __forceinline__ double bf16_hi(uint32_t v) {
  return (double)__uint_as_float(v & 0xFFFF0000u);
}

// acc[j] += products of element pair j of the 8 (4 independent chains).
__device__ __forceinline__ void dot8_bf16(u32x4 a, u32x4 b, double (&acc)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[i] = fma(bf16_lo(a[i]), bf16_lo(b[i]), acc[i]);
    acc[i] = fma(bf16_hi(a[i]), bf16_hi(b[i]), acc[i]);
  }
}

// DPP reductions over the 64 lanes (row_shr 1,2,4,8, then row_bcast 15 and
// 31); the result of lane 63 is returned to every lane. Lanes without a DPP
// source keep their own value.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = __double2loint(v), hi = __double2hiint(v);
  return __hiloint2double(dpp<CTRL, ROWS>(hi), dpp<CTRL, ROWS>(lo));
}

__device__ __forceinline__ double wave_max(double v) {
  v = fmax(v, dpp_d<0x111, 0xf>(v));
  v = fmax(v, dpp_d<0x112, 0xf>(v));
  v = fmax(v, dpp_d<0x114, 0xf>(v));
  v = fmax(v, dpp_d<0x118, 0xf>(v));
  v = fmax(v, dpp_d<0x142, 0xa>(v));
  v = fmax(v, dpp_d<0x143, 0xc>(v));
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ int wave_min(int v) {
  v = min(v, dpp<0x111, 0xf>(v));
  v = min(v, dpp<0x112, 0xf>(v));
  v = min(v, dpp<0x114, 0xf>(v));
  v = min(v, dpp<0x118, 0xf>(v));
  v = min(v, dpp<0x142, 0xa>(v));
  v = min(v, dpp<0x143, 0xc>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the 64 lanes in a fixed DPP tree (lanes without a source add 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d0(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS,
                                             0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS,
                                             0xf, false);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_d0<0x111, 0xf>(v);
  v += dpp_d0<0x112, 0xf>(v);
  v += dpp_d0<0x114, 0xf>(v);
  v += dpp_d0<0x118, 0xf>(v);
  v += dpp_d0<0x142, 0xa>(v);
  v += dpp_d0<0x143, 0xc>(v);
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  return __hiloint2double(hi, lo);
}

constexpr int kRouterWaves = 4;
constexpr int kRouterCPL = 16;  // 16-byte chunks per lane in flight

__global__ __launch_bounds__(kRouterWaves * 64) void router_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ R, int hidden,
    int n, double *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kRouterWaves + wave_id();
  const int t = blockIdx.y;
  if (e >= n) return;  // whole wave; no barrier below
  gu4_t *Rr = (gu4_t *)(R + (size_t)e * hidden);
  gu4_t *xr = (gu4_t *)(x + (size_t)t * hidden);
  const int nchunk = hidden / 8;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = 0; c0 < nchunk; c0 += 64 * kRouterCPL) {
    // Every lane loads (at a clamped index) so that all loads issue before
    // the first use; lanes past the row's end then use zeros.
    u32x4 rv[kRouterCPL], xv[kRouterCPL];
#pragma unroll
    for (int i = 0; i < kRouterCPL; ++i) {
      if (c0 + 64 * i >= nchunk) break;  // wave-uniform
      const int c = min(c0 + lane + 64 * i, nchunk - 1);
      rv[i] = Rr[c];
      xv[i] = xr[c];
    }
#pragma unroll
    for (int i = 0; i < kRouterCPL; ++i) {
      if (c0 + 64 * i >= nchunk) break;
      const bool ok = c0 + lane + 64 * i < nchunk;
      const u32x4 z = {0u, 0u, 0u, 0u};
      dot8_bf16(ok ? rv[i] : z, ok ? xv[i] : z, acc);
    }
  }
  const double total = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
  if (lane == 0) logits[(size_t)t * n + e] = total;
}

__device__ __forceinline__ double sigmoid_d(double v) {
  return 1.0 / (1.0 + exp(-v));
}


__device__ __forceinline__ double readlane_d(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}

// Order-preserving map of fp32 bits to uint32 (larger float -> larger int).
__device__ __forceinline__ uint32_t f32_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_unorder(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Round-based selection over the lane-resident keys (k wave-wide arg-max
// rounds); the slow path, used when the candidate filter below keeps more
// than 64 keys. Returns this lane's selection for rank `lane` (< k).
template <int KPL>
__device__ __forceinline__ void topk_rounds(const double (&key)[KPL],
                                            uint64_t avail, int k, int lane,
                                            int *sel, double *sel_key) {
  for (int r = 0; r < k; ++r) {
    double bk = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (((avail >> i) & 1) && (bi < 0 || key[i] > bk)) {
        bk = key[i];
        bi = i;
      }
    const double m = wave_max(bk);
    int win = wave_min((bi >= 0 && bk == m) ? lane + 64 * bi : INT_MAX);
    if (win == INT_MAX)
      win = wave_min(avail ? lane + 64 * (int)__builtin_ctzll(avail) : INT_MAX);
    if ((win & 63) == lane) avail &= ~(1ull << (win >> 6));
    if (lane == r) {
      *sel = win;
      *sel_key = m;
    }
  }
}

// One wave per token. Expert e's key lives in lane e % 64, slot e / 64.
//  1. tau = the k-th largest of the 64 lane maxima (rounded down to fp32),
//     found bit by bit with ballot counts: at least k keys are >= tau, so
//     the top k are among the keys >= tau (typically ~18 of 896).
//  2. Those candidates are compacted to one per lane (mbcnt offsets), in
//     ascending expert index.
//  3. Each candidate's rank = number of candidates with a higher key, or an
//     equal key and a lower index; ranks < k are the selection, in order.
// Exactly the sort-by-(key desc, index asc) selection; no sequential rounds.
// NaN keys rank below every number.
template <int KPL, typename LT>
__global__ __launch_bounds__(64) void topk_kernel(const LT *__restrict__ logits,
                                                  const float *__restrict__ bias,
                                                  int n, int k,
                                                  int32_t *__restrict__ idx,
                                                  float *__restrict__ w) {
  __shared__ double cand_key[64];
  __shared__ int cand_idx[64];
  __shared__ double ranked[K3_MAX_TOPK];
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  const LT *L = logits + (size_t)t * n;
  LT raw[KPL];
  float b[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) raw[i] = L[min(lane + 64 * i, n - 1)];
  if (bias) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) b[i] = bias[min(lane + 64 * i, n - 1)];
  }
  double key[KPL];
  uint64_t avail = 0;
  double lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const double l = (double)raw[i];
    double kv = bias ? sigmoid_d(l) + (double)b[i] : l;
    if (kv != kv) kv = -INFINITY;  // NaN ranks below every number
    key[i] = kv;
    if (lane + 64 * i < n) {
      avail |= 1ull << i;
      lmax = fmax(lmax, kv);
    }
  }
  // 1. k-th largest lane maximum (fp32, rounded down), MSB-first search.
  const uint32_t um = f32_order(__double2float_rd(lmax));
  uint32_t pre = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = pre | (1u << bit);
    if (__popcll(__ballot(um >= c)) >= k) pre = c;
  }
  const double tau = (double)f32_unorder(pre);
  // 2. candidates (key >= tau), positions in ascending expert index
  int base = 0;
  int my_pos[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const bool c = ((avail >> i) & 1) && key[i] >= tau;
    const uint64_t m = __ballot(c);
    my_pos[i] = c ? base + (int)__builtin_amdgcn_mbcnt_hi(
                               (uint32_t)(m >> 32),
                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0))
                  : -1;
    base += __popcll(m);
  }
  const int C = base;
  int sel = 0;
  double sel_key = 0.0;
  if (C <= 64) {
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (my_pos[i] >= 0) {
        cand_key[my_pos[i]] = key[i];
        cand_idx[my_pos[i]] = lane + 64 * i;
      }
    __syncthreads();
    const double ck = lane < C ? cand_key[lane] : -INFINITY;
    const int ci = lane < C ? cand_idx[lane] : INT_MAX;
    int rank = 0;
    for (int j = 0; j < C; ++j) {
      const double kj = readlane_d(ck, j);
      const int ij = __builtin_amdgcn_readlane(ci, j);
      rank += (kj > ck || (kj == ck && ij < ci)) ? 1 : 0;
    }
    __syncthreads();
    if (lane < C && rank < k) {
      cand_idx[rank] = ci;  // every lane has read its candidate already
      cand_key[rank] = ck;
    }
    __syncthreads();
    if (lane < k) {
      sel = cand_idx[lane];
      sel_key = cand_key[lane];
    }
  } else {
    topk_rounds<KPL>(key, avail, k, lane, &sel, &sel_key);
  }
  // weights from the unbiased scores, renormalised, summed in rank order
  double logit = sel_key;  // without a bias the key is the logit itself
  if (bias && lane < k) logit = (double)L[sel];
  const double s = lane < k ? sigmoid_d(logit) : 0.0;
  if (lane < k) ranked[lane] = s;
  __syncthreads();
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += ranked[j];
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel;
    w[(size_t)t * k + lane] = (float)(s / sum);
  }
}

template <typename LT>
hipError_t launch_topk(const LT *logits, const float *bias, int T, int n,
                       int k, int32_t *idx, float *w, hipStream_t s) {
  const int kpl = (n + 63) / 64;
#define K3_TOPK_CASE(KPL)                                                      \
  if (kpl <= KPL) {                                                            \
    hipLaunchKernelGGL((topk_kernel<KPL, LT>), dim3(T), dim3(64), 0, s,       \
                       logits, bias, n, k, idx, w);                            \
    return hipGetLastError();                                                  \
  }
  K3_TOPK_CASE(1)
  K3_TOPK_CASE(2)
  K3_TOPK_CASE(4)
  K3_TOPK_CASE(8)
  K3_TOPK_CASE(16)
  K3_TOPK_CASE(32)
  K3_TOPK_CASE(64)
#undef K3_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_router(const uint16_t *x, const uint16_t *R, int T,
                         int hidden, int n, double *logits, hipStream_t s) {
  hipLaunchKernelGGL(router_kernel,
                     dim3((n + kRouterWaves - 1) / kRouterWaves, T),
                     dim3(kRouterWaves * 64), 0, s, x, R, hidden, n, logits);
  return hipGetLastError();
}

hipError_t launch_topk_f64(const double *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s) {
  return launch_topk(logits, bias, T, n, k, idx, w, s);
}

hipError_t launch_topk_f32(const float *logits, const float *bias, int T,
                           int n, int k, int32_t *idx, float *w,
                           hipStream_t s) {
  return launch_topk(logits, bias, T, n, k, idx, w, s);
}

}  // namespace k3
