// Batched decode and prefill: the token->expert permutation and the
// per-token weighted combine. (The grouped products: k3_batched_mfma.hip for
// decode batches, k3_prefill.hip for prefill.)
//
// The T*k routing pairs (t, j) are sorted by expert, stably by pair index
// (token, then slot), so every expert's tokens form one contiguous run. A
// run is cut into work items of at most item_tok tokens, the column count of
// the kernels that multiply them.
#include "k3_stream.h"

namespace k3 {

namespace {

constexpr int kPermThreads = 1024;

// Inclusive prefix sum over the block's 1024 threads (wave scans + LDS).
__device__ int block_scan_incl(int v, int *tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  if (w == 0) {
    int s = lane < kPermThreads / 64 ? tmp[lane] : 0;
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(s, d);
      if (lane >= d) s += u;
    }
    if (lane < kPermThreads / 64) tmp[lane] = s;
  }
  __syncthreads();
  const int r = v + (w > 0 ? tmp[w - 1] : 0);
  __syncthreads();
  return r;
}

// One workgroup. Pairs p = t*k + j with expert idx[p]; entries outside
// [0, n) are not placed (they are counted in *n_bad).
//   counts[e], offsets[e]        run length and start of expert e
//   pair_token[q], pair_slot[q]  the q-th pair in (expert, pair index) order
//   pair_pos[p]                  q of pair p (-1 when not placed)
//   items: item_e/off/cnt[i]     expert, first q, tokens (<= item_tok)
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t *__restrict__ idx, int T, int k, int n,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ pair_token, int32_t *__restrict__ pair_slot,
    int32_t *__restrict__ pair_pos, int32_t *__restrict__ item_e,
    int32_t *__restrict__ item_off, int32_t *__restrict__ item_cnt,
    int32_t *__restrict__ n_items, int32_t *__restrict__ n_bad, int item_tok, int pack_tok) {
  __shared__ int cnt[K3_MAX_EXPERTS];
  __shared__ int start[K3_MAX_EXPERTS];  // offsets, then running fill base
  __shared__ unsigned long long mask[K3_MAX_EXPERTS];
  __shared__ int chunk_e[kPermThreads];
  __shared__ int tmp[kPermThreads / 64];
  __shared__ int bad, chunk_slow, n_large;
  const int tid = threadIdx.x;
  const int P = T * k;
  for (int e = tid; e < n; e += kPermThreads) cnt[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kPermThreads) {
    const int e = idx[p];
    if (e >= 0 && e < n)
      atomicAdd(&cnt[e], 1);
    else
      atomicAdd(&bad, 1);
  }
  __syncthreads();
  // exclusive scan of cnt over experts: each thread owns a contiguous span
  const int per = (n + kPermThreads - 1) / kPermThreads;
  const int e0 = min(n, tid * per), e1 = min(n, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += cnt[e];
  int run = block_scan_incl(local, tmp) - local;
  for (int e = e0; e < e1; ++e) {
    start[e] = run;
    counts[e] = cnt[e];
    offsets[e] = run;
    run += cnt[e];
  }
  __syncthreads();
  // Stable placement, 64 tokens at a time. Fast path: bit t of mask[e] says
  // token t0+t chose e, so a pair's rank among its expert's pairs is start[e]
  // plus the chosen bits below its token. A token that names an expert twice
  // (never the case for top-k output) or an entry outside [0, n) sends the
  // chunk to the exact path, which counts earlier equal entries one by one.
  for (int t0 = 0; t0 < T; t0 += 64) {
    const int tn = min(64, T - t0);
    const int c = t0 * k, cP = tn * k;  // this chunk's pairs [c, c + cP)
    for (int e = tid; e < n; e += kPermThreads) mask[e] = 0ull;
    if (tid == 0) chunk_slow = 0;
    __syncthreads();
    for (int i = tid; i < cP; i += kPermThreads) {
      const int e = idx[c + i];
      if (e >= 0 && e < n) {
        const unsigned long long bit = 1ull << (i / k);
        if (atomicOr(&mask[e], bit) & bit) chunk_slow = 1;
      } else {
        chunk_slow = 1;
      }
    }
    __syncthreads();
    if (!chunk_slow) {
      for (int i = tid; i < cP; i += kPermThreads) {
        const int p = c + i, e = idx[p], tl = i / k;
        const int q = start[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
        pair_token[q] = p / k;
        pair_slot[q] = p % k;
        pair_pos[p] = q;
      }
      __syncthreads();
      for (int e = tid; e < n; e += kPermThreads) start[e] += __popcll(mask[e]);
      __syncthreads();
      continue;
    }
    for (int b = 0; b < cP; b += kPermThreads) {
      const int p = c + b + tid;
      const int e = b + tid < cP ? idx[p] : -1;
      const bool ok = e >= 0 && e < n;
      chunk_e[tid] = ok ? e : -1;
      __syncthreads();
      if (ok) {
        int r = 0;
        for (int i = 0; i < tid; ++i) r += chunk_e[i] == e;
        const int q = start[e] + r;
        pair_token[q] = p / k;
        pair_slot[q] = p % k;
        pair_pos[p] = q;
      } else if (b + tid < cP) {
        pair_pos[p] = -1;
      }
      __syncthreads();
      // advance each expert's base by its pairs here (its last entry writes)
      if (ok) {
        bool last = true;
        for (int i = tid + 1; i < kPermThreads; ++i)
          if (chunk_e[i] == e) {
            last = false;
            break;
          }
        if (last) {
          int r = 0;
          for (int i = 0; i <= tid; ++i) r += chunk_e[i] == e;
          start[e] += r;
        }
      }
      __syncthreads();
    }
  }
  // work items: ceil(cnt/tok) per expert; those of more than pack pairs
  // first, then the others, each class in expert order. ni[0] = all items,
  // ni[1] = the first class's.
  auto cut = [&](int tok, int pack, int32_t *ie, int32_t *ioff, int32_t *icnt, int32_t *ni) {
    int nl = 0, ns = 0;
    for (int e = e0; e < e1; ++e)
      for (int s = 0; s < cnt[e]; s += tok) (min(tok, cnt[e] - s) > pack ? nl : ns) += 1;
    const int lb = block_scan_incl(nl, tmp) - nl;
    const int sb = block_scan_incl(ns, tmp) - ns;
    if (tid == kPermThreads - 1) n_large = lb + nl;
    __syncthreads();
    int il = lb, is = n_large + sb;
    for (int e = e0; e < e1; ++e) {
      const int off = offsets[e];
      for (int s = 0; s < cnt[e]; s += tok) {
        const int c = min(tok, cnt[e] - s);
        const int at = c > pack ? il++ : is++;
        ie[at] = e;
        ioff[at] = off + s;
        icnt[at] = c;
      }
    }
    if (tid == kPermThreads - 1) {
      ni[0] = is;
      ni[1] = n_large;
    }
  };
  cut(item_tok, pack_tok, item_e, item_off, item_cnt, n_items);
  if (tid == 0) *n_bad = bad;
}

struct Items {
  const int32_t *e, *off, *cnt, *n;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Y[t][i] = sum_j w[t][j] * yp[pair_pos[t*k + j]][i] in rank order j, fp32,
// then bf16 (RNE); four consecutive columns per thread (16-byte loads and
// stores). hidden % 32 == 0, and yp, Y and Y32 are 16-byte aligned (the ABI
// refuses other outputs). Tokens past the grid's y extent are taken in
// strides of it.
__global__ __launch_bounds__(256) void combine_batched_kernel(
    const float *__restrict__ yp, const float *__restrict__ w,
    const int32_t *__restrict__ pair_pos, int k, int hidden, int T,
    uint16_t *__restrict__ Y, float *__restrict__ Y32) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= hidden) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {  // tokens past the grid's y extent
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j0 = 0; j0 < k; j0 += 16) {  // issue a batch of loads, then add
      f32x4 v[16];  // partials are read once: non-temporal
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[j] = j0 + j < k ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(
                                yp + (size_t)pair_pos[(size_t)t * k + j0 + j] * hidden + i))
                          : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < k) {
          const float wj = w[(size_t)t * k + j0 + j];
          a0 = fmaf(wj, v[j].x, a0);
          a1 = fmaf(wj, v[j].y, a1);
          a2 = fmaf(wj, v[j].z, a2);
          a3 = fmaf(wj, v[j].w, a3);
        }
    }
    const size_t o = (size_t)t * hidden + i;
    if (Y32) *reinterpret_cast<float4 *>(Y32 + o) = float4{a0, a1, a2, a3};
    if (Y) {
      const uint32_t lo = f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
      const uint32_t hi = f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
      *reinterpret_cast<uint2 *>(Y + o) = uint2{lo, hi};
    }
  }
}

}  // namespace

hipError_t launch_permute(const int32_t *idx, int T, int k, int n,
                          const PermOut &o, int item_tok, int pack_tok, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, idx, T,
                     k, n, o.counts, o.offsets, o.pair_token, o.pair_slot,
                     o.pair_pos, o.item_e, o.item_off, o.item_cnt, o.n_items,
                     o.n_bad, item_tok, pack_tok);
  return hipGetLastError();
}

hipError_t launch_combine_batched(const float *yp, const float *w,
                                  const int32_t *pair_pos, int T, int k,
                                  int hidden, uint16_t *Y, float *Y32,
                                  hipStream_t s) {
  const unsigned gy = (unsigned)(T < 65535 ? T : 65535);
  hipLaunchKernelGGL(combine_batched_kernel, dim3((hidden / 4 + 255) / 256, gy), dim3(256), 0,
                     s, yp, w, pair_pos, k, hidden, T, Y, Y32);
  return hipGetLastError();
}

}  // namespace k3
