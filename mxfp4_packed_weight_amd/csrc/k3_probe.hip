// Calibration read: the rate at which this device streams a large buffer
// from HBM with plain 16-byte loads, the yardstick the expert kernels'
// rates are also reported against. Every byte is read once (non-temporal),
// folded into a per-thread XOR so the loads cannot be dropped; `sink` is
// written only if the fold of a block equals a fixed value, which for
// ordinary data essentially never happens.
#include "k3_internal.h"

namespace k3 {

namespace {

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;

// Grid-stride over n 16-byte units, kProbeUnroll loads in flight per lane.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(
    const u32v4 *__restrict__ p, size_t n, uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
    u32v4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32v4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
  const unsigned grid = (unsigned)num_cus();  // one 512-thread workgroup per compute unit
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, s,
                     static_cast<const u32v4 *>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace k3
