// Wave-level helpers and the top-k selection of one token by one wave,
// shared by the router's top-k kernel and the fused decode kernels.
//
// One wave per token. Expert e's key lives in lane e % 64, slot e / 64.
//  1. tau = the k-th largest of the 64 lane maxima (rounded down to fp32),
//     found bit by bit with ballot counts: at least k keys are >= tau, so
//     the top k are among the keys >= tau (typically ~18 of 896).
//  2. Those candidates are packed into LDS (per-lane counts, a prefix sum
//     from ballots of the count bits).
//  3. Each candidate's rank = number of candidates with a higher key, or an
//     equal key and a lower index; ranks < k are the selection, in order.
// Exactly the sort-by-(key desc, index asc) selection. topk_wg does the
// same with a whole workgroup, one expert per thread, for the decode layer,
// where every workgroup waits for the selection. NaN keys rank below every
// number. The
// routing bias only changes the keys; the weights always come from the
// unbiased sigmoid scores ([ZOR] "How is the C engine actually built?",
// invariant 3), renormalised to sum to one, summed in rank order.
#pragma once

#include <limits.h>
#include <math.h>

#include "k3_decode.h"
#include "k3_internal.h"

namespace k3 {

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

// Orders this wave's LDS writes before its later LDS reads (one wave only).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Top-k of one token's n logits held in registers by one wave: raw[i] is the
// logit of expert lane + 64 i (entries at or past n are ignored). On return
// lanes < k hold the j-th selection in *sel_out and its renormalised weight
// times `scale` in *wt_out (rank order). `tk` is the wave's LDS scratch; with
// a bias, logit_of(e) returns expert e's logit (the weights use unbiased
// scores).
template <int KPL, typename LT, class LogitOf>
__device__ __forceinline__ void topk_core(const LT (&raw)[KPL],
                                          const float *__restrict__ bias, int n,
                                          int k, TopkLds &tk, LogitOf logit_of,
                                          int *sel_out, float *wt_out,
                                          double scale = 1.0) {
  const int lane = threadIdx.x & 63;
  float b[KPL];
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
  // 1. tau = k-th largest lane maximum (fp32, rounded down), MSB first.
  const uint32_t um = f32_order(__double2float_rd(lmax));
  uint32_t pre = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = pre | (1u << bit);
    if ((int)__popcll(__ballot(um >= c)) >= k) pre = c;
  }
  const double tau = (double)f32_unorder(pre);
  // 2. candidates (key >= tau): per-lane count, exclusive prefix over lanes
  //    from one ballot per count bit, then packed into LDS.
  uint64_t cmask = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i)
    if (((avail >> i) & 1) && key[i] >= tau) cmask |= 1ull << i;
  const int cnt = __popcll(cmask);
  int base = 0, C = 0;
#pragma unroll
  for (int bit = 0; bit < 7; ++bit) {  // cnt <= KPL <= 64
    const uint64_t m = __ballot((cnt >> bit) & 1);
    base += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0))
            << bit;
    C += __popcll(m) << bit;
  }
  int sel = 0;
  double sel_key = 0.0;
  if (C <= 64) {
    int at = base;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if ((cmask >> i) & 1) {
        tk.cand_key[at] = key[i];
        tk.cand_idx[at] = lane + 64 * i;
        ++at;
      }
    wave_lds_sync();
    const double ck = lane < C ? tk.cand_key[lane] : -INFINITY;
    const int ci = lane < C ? tk.cand_idx[lane] : INT_MAX;
    int rank = 0;
    for (int j = 0; j < C; ++j) {
      const double kj = readlane_d(ck, j);
      const int ij = __builtin_amdgcn_readlane(ci, j);
      rank += (kj > ck || (kj == ck && ij < ci)) ? 1 : 0;
    }
    wave_lds_sync();
    if (lane < C && rank < k) {
      tk.cand_idx[rank] = ci;  // every lane has read its candidate already
      tk.cand_key[rank] = ck;
    }
    wave_lds_sync();
    if (lane < k) {
      sel = tk.cand_idx[lane];
      sel_key = tk.cand_key[lane];
    }
  } else {
    topk_rounds<KPL>(key, avail, k, lane, &sel, &sel_key);
  }
  // weights from the unbiased scores, renormalised, summed in rank order
  double logit = sel_key;  // without a bias the key is the logit itself
  if (bias && lane < k) logit = logit_of(sel);
  const double s = lane < k ? sigmoid_d(logit) : 0.0;
  if (lane < k) tk.ranked[lane] = s;
  wave_lds_sync();
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += tk.ranked[j];
  *sel_out = sel;
  *wt_out = (float)((s / sum) * scale);
}

// The same with the logits read from memory (L[e], e < n).
template <int KPL, typename LT>
__device__ __forceinline__ void topk_wave(const LT *__restrict__ L,
                                          const float *__restrict__ bias, int n,
                                          int k, TopkLds &tk, int *sel_out,
                                          float *wt_out, double scale = 1.0) {
  const int lane = threadIdx.x & 63;
  LT raw[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) raw[i] = L[min(lane + 64 * i, n - 1)];
  topk_core<KPL, LT>(raw, bias, n, k, tk, [&](int e) { return (double)L[e]; },
                     sel_out, wt_out, scale);
}

// Weights of a ranked selection (s.sel_key, rank order) in one wave: the
// scores renormalised, summed in rank order (as topk_core without a bias:
// the key is the logit).
__device__ __forceinline__ void topk_wg_weights_wave(TopkWgLds &s, int k) {
  const int lane = threadIdx.x & 63;
  const double sc = lane < k ? sigmoid_d(s.sel_key[lane]) : 0.0;
  if (lane < k) s.ranked[lane] = sc;
  wave_lds_sync();
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += s.ranked[j];
  if (lane < k) s.wt[lane] = (float)(sc / sum);
}

// Top-k of one token's n <= blockDim logits by a whole workgroup (16 waves),
// one expert per thread: the selection and weights of topk_core, with the
// three steps spread over the waves so that no single wave walks the keys.
//   1. tau: the k-th largest of the 64 column maxima (column = e % 64):
//      each wave computes the maxima, compares every column with 4 others
//      and adds its counts into LDS; the column with fewer than k above it
//      and at least k at or above it holds tau.
//   2. candidates (key >= tau) are packed per wave with ballots, wave
//      offsets from LDS.
//   3. each wave ranks every candidate against 4 others; the counts add up
//      in LDS to the exact (key desc, index asc) rank.
// More than 64 candidates (many equal keys) take topk_core on wave 0.
// Result in s.sel / s.wt (rank order, lanes < k) after a barrier. With
// kWeights false the weights may be left to topk_wg_weights, so that a
// caller can start on the selected experts first.
template <int NWAVES, bool kWeights = true>
__device__ __forceinline__ void topk_wg(const double *__restrict__ L, int n, int k, TopkWgLds &s) {
  static_assert(NWAVES * 4 >= 64, "each wave compares against 4 columns");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  double key = -INFINITY;
  if (t < n) {
    key = L[t];
    if (key != key) key = -INFINITY;  // NaN ranks below every number
  }
  s.okey[t] = f32_order(__double2float_rd(key));
  if (t < 64) {
    s.gt[t] = 0;
    s.ge[t] = 0;
    s.rank[t] = 0;
  }
  __syncthreads();
  // 1. column maxima (each wave, redundantly), then 4 comparisons per lane.
  uint32_t col[NWAVES];
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) col[i] = s.okey[lane + 64 * i];
  __builtin_amdgcn_sched_barrier(0);  // every read in flight before the first use
  uint32_t um = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) um = max(um, col[i]);
  {
    int gt = 0, ge = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = __builtin_amdgcn_readlane(um, 4 * w + j);
      gt += v > um ? 1 : 0;
      ge += v >= um ? 1 : 0;
    }
    atomicAdd(&s.gt[lane], gt);
    atomicAdd(&s.ge[lane], ge);
  }
  __syncthreads();
  const uint64_t holds = __ballot(s.gt[lane] < k && s.ge[lane] >= k);
  const double tau = (double)f32_unorder(
      __builtin_amdgcn_readlane(um, (int)__builtin_ctzll(holds)));
  // 2. candidates, packed in wave order.
  const bool cand = t < n && key >= tau;
  const uint64_t m = __ballot(cand);
  if (lane == 0) s.wave_cnt[w] = __popcll(m);
  __syncthreads();
  int base = 0, C = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    const int c = s.wave_cnt[i];
    base += i < w ? c : 0;
    C += c;
  }
  if (C <= 64) {
    if (cand) {
      const int at = base + (int)__builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(m >> 32),
                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      s.cand_key[at] = key;
      s.cand_idx[at] = t;
    }
    __syncthreads();
    // 3. candidate `lane` against candidates 4w .. 4w + 3.
    if (lane < C) {
      const double ck = s.cand_key[lane];
      const int ci = s.cand_idx[lane];
      double kq[4];
      int iq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // slots past C hold stale bytes, never used
        kq[j] = s.cand_key[min(4 * w + j, 63)];
        iq[j] = s.cand_idx[min(4 * w + j, 63)];
      }
      __builtin_amdgcn_sched_barrier(0);  // every read in flight before the first use
      int r = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * w + j < C) r += (kq[j] > ck || (kq[j] == ck && iq[j] < ci)) ? 1 : 0;
      if (r) atomicAdd(&s.rank[lane], r);
    }
    __syncthreads();
    if (w == 0) {
      if (lane < C) {
        const int r = s.rank[lane];
        if (r < k) {
          s.sel[r] = s.cand_idx[lane];
          s.sel_key[r] = s.cand_key[lane];
        }
      }
      wave_lds_sync();
      if constexpr (kWeights) topk_wg_weights_wave(s, k);
      if (lane == 0) s.wt_later = kWeights ? 0 : 1;
    }
  } else if (w == 0) {
    int e;
    float wt;
    topk_wave<kFusedTopkMaxExperts / 64, double>(L, nullptr, n, k, s.tk, &e, &wt);
    if (lane < k) {
      s.sel[lane] = e;
      s.wt[lane] = wt;
    }
    if (lane == 0) s.wt_later = 0;
  }
  __syncthreads();
}

// The weights of topk_wg's selection in the calling wave's registers: lane
// j < k returns rank j's weight, computed here when topk_wg left them (the
// same operations and order as topk_wg_weights_wave), else read from s.wt.
// Any wave, any time after topk_wg returned; LDS is only read.
__device__ __forceinline__ float topk_wg_weight_lane(const TopkWgLds &s, int k) {
  const int lane = threadIdx.x & 63;
  if (!s.wt_later) return lane < k ? s.wt[lane] : 0.f;
  const double sc = lane < k ? sigmoid_d(s.sel_key[lane]) : 0.0;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += readlane_d(sc, j);
  return lane < k ? (float)(sc / sum) : 0.f;
}

}  // namespace k3
