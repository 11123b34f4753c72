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
constexpr int kPermCache = 32;  // chunks whose entries a thread can hold in registers
constexpr int kPermMaxChunks = 256;  // chunks placed by workgroups of their own, at most

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

// Stable placement of one chunk of 64 tokens (pairs [c, c + cP)), given
// start[e] in LDS = the position of expert e's first pair of the chunk;
// advances start[] past the chunk's pairs. Every thread of the workgroup
// takes part; entry(i) is the expert of pair c + i (a thread asks only for
// the i it owns: i = tid + 1024 j). Fast path: bit t of mask[e] says token
// t chose e, so a pair's rank among its expert's pairs is start[e] plus the
// chosen bits below its token. A token that names an expert twice (never the
// case for top-k output) or an entry outside [0, n) sends the chunk to the
// exact path, which counts earlier equal entries one by one. The barriers
// order LDS only: the pairs' stores need not be complete before the next
// chunk (nothing here reads them).
template <class Entry>
__device__ __forceinline__ void place_chunk(Entry entry, int c, int cP, int k, int n, int *start,
                                            unsigned long long *mask, int *chunk_e,
                                            int &chunk_slow, int32_t *__restrict__ pair_token,
                                            int32_t *__restrict__ pair_slot,
                                            int32_t *__restrict__ pair_pos) {
  const int tid = threadIdx.x;
  for (int e = tid; e < n; e += kPermThreads) mask[e] = 0ull;
  if (tid == 0) chunk_slow = 0;
  lds_barrier();
  for (int i = tid; i < cP; i += kPermThreads) {
    const int e = entry(i);
    if (e >= 0 && e < n) {
      const unsigned long long bit = 1ull << (i / k);
      if (atomicOr(&mask[e], bit) & bit) chunk_slow = 1;
    } else {
      chunk_slow = 1;
    }
  }
  lds_barrier();
  if (!chunk_slow) {
    for (int i = tid; i < cP; i += kPermThreads) {
      const int p = c + i, e = entry(i), tl = i / k;
      const int q = start[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
      pair_token[q] = p / k;
      pair_slot[q] = p % k;
      pair_pos[p] = q;
    }
    lds_barrier();
    for (int e = tid; e < n; e += kPermThreads) start[e] += __popcll(mask[e]);
    lds_barrier();
    return;
  }
  for (int b = 0; b < cP; b += kPermThreads) {
    const int p = c + b + tid;
    const int e = b + tid < cP ? entry(b + tid) : -1;
    const bool ok = e >= 0 && e < n;
    chunk_e[tid] = ok ? e : -1;
    lds_barrier();
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
    lds_barrier();
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
    lds_barrier();
  }
}

// Work items: ceil(cnt/tok) per expert, from cnt[] (LDS) and offsets[]
// (written by this workgroup); those of more than pack pairs first, then
// the others, each class in expert order. ni[0] = all items, ni[1] = the
// first class's. Thread tid owns experts [e0, e1).
__device__ __forceinline__ void cut_items(const int *cnt, const int32_t *offsets, int e0, int e1,
                                          int tok, int pack, int *tmp, int &n_large,
                                          int32_t *__restrict__ ie, int32_t *__restrict__ ioff,
                                          int32_t *__restrict__ icnt, int32_t *__restrict__ ni) {
  const int tid = threadIdx.x;
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
}

// The permutation. Pairs p = t*k + j with expert idx[p]; entries outside
// [0, n) are not placed (they are counted in *n_bad).
//   counts[e], offsets[e]        run length and start of expert e
//   pair_token[q], pair_slot[q]  the q-th pair in (expert, pair index) order
//   pair_pos[p]                  q of pair p (-1 when not placed)
//   items: item_e/off/cnt[i]     expert, first q, tokens (<= item_tok)
// permute_kernel does it all in one workgroup, a chunk of 64 tokens at a
// time. For many chunks the chunks go to workgroups of their own in three
// launches instead: perm_count_kernel (each chunk's pairs per expert),
// perm_scan_kernel (one workgroup: runs, offsets, each chunk's start per
// expert, items) and perm_place_kernel (each chunk placed from its starts).
// The positions are the same.
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
  // When a chunk of 64 tokens has at most one pair per thread and there are
  // at most kPermCache chunks, each thread loads its pair of every chunk
  // once, here: ec[c] is entry 64 k c + tid. The chunk loop then reads no
  // global memory, so its waits do not wait for its stores either.
  const int nchunks = (T + 63) / 64;
  const bool cached = 64 * k <= kPermThreads && nchunks <= kPermCache;
  int ec[kPermCache];
  if (cached) {
#pragma unroll
    for (int c = 0; c < kPermCache; ++c)
      ec[c] = c < nchunks && tid < min(64, T - 64 * c) * k ? idx[64 * k * c + tid] : 0;
#pragma unroll
    for (int c = 0; c < kPermCache; ++c)
      if (c < nchunks && tid < min(64, T - 64 * c) * k) {
        if (ec[c] >= 0 && ec[c] < n)
          atomicAdd(&cnt[ec[c]], 1);
        else
          atomicAdd(&bad, 1);
      }
  } else {
    for (int p = tid; p < P; p += kPermThreads) {
      const int e = idx[p];
      if (e >= 0 && e < n)
        atomicAdd(&cnt[e], 1);
      else
        atomicAdd(&bad, 1);
    }
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
  // one loop instance per case, so that the cached one holds no global load
  if (cached) {
    for (int t0 = 0; t0 < T; t0 += 64) {
      place_chunk([&](int) { return ec[0]; }, t0 * k, min(64, T - t0) * k, k, n, start, mask,
                  chunk_e, chunk_slow, pair_token, pair_slot, pair_pos);
#pragma unroll
      for (int j = 0; j + 1 < kPermCache; ++j) ec[j] = ec[j + 1];
    }
  } else {
    for (int t0 = 0; t0 < T; t0 += 64) {
      const int c = t0 * k;
      place_chunk([&](int i) { return idx[c + i]; }, c, min(64, T - t0) * k, k, n, start, mask,
                  chunk_e, chunk_slow, pair_token, pair_slot, pair_pos);
    }
  }
  cut_items(cnt, offsets, e0, e1, item_tok, pack_tok, tmp, n_large, item_e, item_off, item_cnt,
            n_items);
  if (tid == 0) *n_bad = bad;
}

// Each chunk's pairs per expert: cs[chunk][e], and its entries outside
// [0, n) in cs[nchunks][chunk]. One workgroup per chunk.
__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(
    const int32_t *__restrict__ idx, int T, int k, int n, int32_t *__restrict__ cs) {
  __shared__ int cnt[K3_MAX_EXPERTS];
  __shared__ int bad;
  const int tid = threadIdx.x, ch = blockIdx.x, nchunks = gridDim.x;
  const int c = 64 * ch * k, cP = min(64, T - 64 * ch) * k;
  for (int e = tid; e < n; e += kPermThreads) cnt[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int i = tid; i < cP; i += kPermThreads) {
    const int e = idx[c + i];
    if (e >= 0 && e < n)
      atomicAdd(&cnt[e], 1);
    else
      atomicAdd(&bad, 1);
  }
  __syncthreads();
  for (int e = tid; e < n; e += kPermThreads) cs[(size_t)ch * n + e] = cnt[e];
  if (tid == 0) cs[(size_t)nchunks * n + ch] = bad;
}

// One workgroup: the runs (counts, offsets), each chunk's start per expert
// (cs[chunk][e] becomes the position of expert e's first pair of the chunk),
// the work items and *n_bad.
__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(
    int n, int nchunks, int32_t *__restrict__ cs, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ item_e, int32_t *__restrict__ item_off,
    int32_t *__restrict__ item_cnt, int32_t *__restrict__ n_items, int32_t *__restrict__ n_bad,
    int item_tok, int pack_tok) {
  __shared__ int cnt[K3_MAX_EXPERTS];
  __shared__ int tmp[kPermThreads / 64];
  __shared__ int n_large;
  const int tid = threadIdx.x;
  const int per = (n + kPermThreads - 1) / kPermThreads;
  const int e0 = min(n, tid * per), e1 = min(n, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) {
    int t = 0;
    for (int ch = 0; ch < nchunks; ++ch) t += cs[(size_t)ch * n + e];
    cnt[e] = t;
    local += t;
  }
  int run = block_scan_incl(local, tmp) - local;
  for (int e = e0; e < e1; ++e) {
    counts[e] = cnt[e];
    offsets[e] = run;
    int at = run;
    for (int ch = 0; ch < nchunks; ++ch) {
      const int v = cs[(size_t)ch * n + e];
      cs[(size_t)ch * n + e] = at;
      at += v;
    }
    run += cnt[e];
  }
  if (tid == 0) {
    int b = 0;
    for (int ch = 0; ch < nchunks; ++ch) b += cs[(size_t)nchunks * n + ch];
    *n_bad = b;
  }
  __syncthreads();
  cut_items(cnt, offsets, e0, e1, item_tok, pack_tok, tmp, n_large, item_e, item_off, item_cnt,
            n_items);
}

// One chunk per workgroup, placed from its starts cs[chunk][e].
__global__ __launch_bounds__(kPermThreads) void perm_place_kernel(
    const int32_t *__restrict__ idx, int T, int k, int n, const int32_t *__restrict__ cs,
    int32_t *__restrict__ pair_token, int32_t *__restrict__ pair_slot,
    int32_t *__restrict__ pair_pos) {
  __shared__ int start[K3_MAX_EXPERTS];
  __shared__ unsigned long long mask[K3_MAX_EXPERTS];
  __shared__ int chunk_e[kPermThreads];
  __shared__ int chunk_slow;
  const int ch = blockIdx.x;
  const int c = 64 * ch * k, cP = min(64, T - 64 * ch) * k;
  for (int e = threadIdx.x; e < n; e += kPermThreads) start[e] = cs[(size_t)ch * n + e];
  __syncthreads();
  place_chunk([&](int i) { return idx[c + i]; }, c, cP, k, n, start, mask, chunk_e, chunk_slow,
              pair_token, pair_slot, pair_pos);
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

int perm_chunk_table_ints(int T) {
  const int nchunks = (T + 63) / 64;
  return nchunks > 1 && nchunks <= kPermMaxChunks ? (nchunks + 1) * K3_MAX_EXPERTS : 0;
}

hipError_t launch_permute(const int32_t *idx, int T, int k, int n,
                          const PermOut &o, int item_tok, int pack_tok, hipStream_t s) {
  const int nchunks = (T + 63) / 64;
  if (o.chunk_table && perm_chunk_table_ints(T) > 0) {
    hipLaunchKernelGGL(perm_count_kernel, dim3(nchunks), dim3(kPermThreads), 0, s, idx, T, k, n,
                       o.chunk_table);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kPermThreads), 0, s, n, nchunks,
                       o.chunk_table, o.counts, o.offsets, o.item_e, o.item_off, o.item_cnt,
                       o.n_items, o.n_bad, item_tok, pack_tok);
    hipLaunchKernelGGL(perm_place_kernel, dim3(nchunks), dim3(kPermThreads), 0, s, idx, T, k, n,
                       o.chunk_table, o.pair_token, o.pair_slot, o.pair_pos);
    return hipGetLastError();
  }
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
