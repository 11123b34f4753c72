// Hand-offs between the workgroups of one launch, without cache flushes.
//
// Data that another workgroup of the same launch reads is written with
// device-coherent stores and read with device-coherent loads (agent-scope
// relaxed atomics, which go past this XCD's L2), and a workgroup announces
// that its data is there only after its own stores have completed, by
// storing the call's value into its arrival slot. No L2 writeback or
// invalidate is issued: on this part each one walks a whole XCD's L2.
//
// Arrival slots hold a per-call value chosen by the host (unique in the
// process), so they never need clearing between calls; leftover memory
// equals a call's value only by a 2^-64 chance. Every wait is bounded:
// one that runs out reports failure instead of hanging the device. The bound
// is a number of polls passed by the caller: kSpinLimit, unless a test has
// lowered it (k3_set_wait_limit) to see that failure reported.
#pragma once

#include "k3_stream.h"

namespace k3 {

constexpr int kSpinLimit = K3_WAIT_LIMIT_DEFAULT;  // polls of one wait (~1 s), then fail

template <typename T>
__device__ __forceinline__ void st_dev(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// This workgroup's stores so far have completed; then its slot takes `val`.
__device__ __forceinline__ void arrive(uint64_t *slots, uint64_t val) {
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's stores are done
  __syncthreads();
  if (threadIdx.x == 0) st_dev(slots + blockIdx.x, val);
}

// Hides where a pointer came from, so that no load through it (scalar
// activation loads in particular, which the compiler may otherwise hoist)
// is scheduled above the wait that precedes this call.
template <typename T>
__device__ __forceinline__ T *after_wait(T *p) {
  asm volatile("" : "+s"(p) : : "memory");
  return p;
}

// One wave: waits until slots[i] == val for all i in [first, first + count).
// False if `limit` polls run out.
__device__ __forceinline__ bool wave_wait_range(const uint64_t *slots,
                                                int first, int count,
                                                uint64_t val, int limit) {
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < limit; ++it) {
    bool ok = true;
    for (int i0 = 0; i0 < count; i0 += 256) {  // four loads in flight per lane
      uint64_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + lane + 64 * q;
        v[q] = i < count ? ld_dev(slots + first + i) : val;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ok &= v[q] == val;
    }
    if (__ballot(!ok) == 0) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// One wave: waits until slots[owner] == val for every lane < count (each
// lane names its own owner). False if `limit` polls run out.
__device__ __forceinline__ bool wave_wait_owners(const uint64_t *slots,
                                                 int owner, int count,
                                                 uint64_t val, int limit) {
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < limit; ++it) {
    const bool mine = lane >= count || ld_dev(slots + owner) == val;
    if (__ballot(!mine) == 0) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Workgroup owning tile t when `total` tiles are cut into contiguous ranges
// over `grid` workgroups (wg_range).
__device__ __forceinline__ int tile_owner(int t, int total, int grid) {
  return (int)(((long long)(t + 1) * grid - 1) / total);
}

}  // namespace k3
