// Re-tiling of canonical MXFP4 bytes into the device tile layout (and back).
// Pure byte movement: bijective on every byte of the canonical matrix, done
// once when weights are loaded, never on the hot path.
#include <string.h>

#include "k3_internal.h"

namespace k3 {

namespace {

// Source row of virtual tile row (t, lane) for a plain matrix.
struct PlainRows {
  const uint8_t *nib, *sc;
  int rows;
  __host__ __device__ bool row(int t, int lane, const uint8_t **n,
                               const uint8_t **s, int *r) const {
    *r = t * kTileRows + lane;
    *n = nib;
    *s = sc;
    return *r < rows;
  }
};

// Gate/up interleave: lanes 0..31 gate rows, 32..63 up rows.
struct GateUpRows {
  const uint8_t *gn, *gs, *un, *us;
  int inter;
  __host__ __device__ bool row(int t, int lane, const uint8_t **n,
                               const uint8_t **s, int *r) const {
    int up;
    gu_lane_row(t, lane, &up, r);
    *n = up ? un : gn;
    *s = up ? us : gs;
    return *r < inter;
  }
};

template <class Src>
__host__ __device__ inline void pack_nib16(const Src &src, const MatLayout &m,
                                           int t, int g, int lane,
                                           uint8_t *tiles) {
  const uint8_t *n, *s;
  int r;
  uint8_t *dst = tiles + (size_t)t * m.tile_bytes + code_offset(g, lane);
  if (g < m.G && src.row(t, lane, &n, &s, &r)) {
    const uint8_t *p = n + (size_t)r * (m.cols / 2) + (size_t)16 * g;
    for (int i = 0; i < 16; ++i) dst[i] = p[i];
  } else {
    for (int i = 0; i < 16; ++i) dst[i] = 0;
  }
}

template <class Src>
__host__ __device__ inline void pack_scale4(const Src &src, const MatLayout &m,
                                            int t, int q, int lane,
                                            uint8_t *tiles) {
  const uint8_t *n, *s;
  int r;
  const bool ok = src.row(t, lane, &n, &s, &r);
  for (int b = 0; b < 4; ++b) {
    const int g = 4 * q + b;
    tiles[(size_t)t * m.tile_bytes + scale_offset(g, lane)] =
        (ok && g < m.G) ? s[(size_t)r * m.G + g] : (uint8_t)0;
  }
}

template <class Src>
void pack_host(const Src &src, const MatLayout &m, uint8_t *tiles) {
  for (int t = 0; t < m.ntiles; ++t)
    for (int lane = 0; lane < kTileRows; ++lane) {
      for (int g = 0; g < 4 * m.G4; ++g) pack_nib16(src, m, t, g, lane, tiles);
      for (int q = 0; q < m.G4; ++q) pack_scale4(src, m, t, q, lane, tiles);
    }
}

// One thread per (tile, slot, lane); slots 0..4*G4-1 move code bytes (zero
// past G), slots 4*G4..5*G4-1 move exponent bytes.
template <class Src>
__global__ void pack_kernel(Src src, MatLayout m, uint8_t *tiles) {
  const size_t per_tile = (size_t)(5 * m.G4) * kTileRows;
  const size_t total = per_tile * m.ntiles;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / per_tile);
    const int rem = (int)(i % per_tile);
    const int slot = rem / kTileRows, lane = rem % kTileRows;
    if (slot < 4 * m.G4)
      pack_nib16(src, m, t, slot, lane, tiles);
    else
      pack_scale4(src, m, t, slot - 4 * m.G4, lane, tiles);
  }
}

__host__ __device__ inline void unpack_one(const uint8_t *tiles,
                                           const MatLayout &m, int r, int g,
                                           uint8_t *nib, uint8_t *sc) {
  const int t = r / kTileRows, lane = r % kTileRows;
  const uint8_t *src = tiles + (size_t)t * m.tile_bytes + code_offset(g, lane);
  uint8_t *dst = nib + (size_t)r * (m.cols / 2) + (size_t)16 * g;
  for (int i = 0; i < 16; ++i) dst[i] = src[i];
  sc[(size_t)r * m.G + g] =
      tiles[(size_t)t * m.tile_bytes + scale_offset(g, lane)];
}

__global__ void unpack_kernel(const uint8_t *tiles, MatLayout m, uint8_t *nib,
                              uint8_t *sc) {
  const size_t total = (size_t)m.rows * m.G;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x)
    unpack_one(tiles, m, (int)(i / m.G), (int)(i % m.G), nib, sc);
}

unsigned grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  return (unsigned)(b < 65536 ? (b ? b : 1) : 65536);
}

}  // namespace

void pack_plain_host(const uint8_t *nib, const uint8_t *sc, int rows, int cols,
                     uint8_t *tiles) {
  pack_host(PlainRows{nib, sc, rows}, mat_layout(rows, cols), tiles);
}

void unpack_plain_host(const uint8_t *tiles, int rows, int cols, uint8_t *nib,
                       uint8_t *sc) {
  const MatLayout m = mat_layout(rows, cols);
  for (int r = 0; r < rows; ++r)
    for (int g = 0; g < m.G; ++g) unpack_one(tiles, m, r, g, nib, sc);
}

void pack_expert_host(const uint8_t *gn, const uint8_t *gs, const uint8_t *un,
                      const uint8_t *us, const uint8_t *dn, const uint8_t *ds,
                      int hidden, int inter, uint8_t *dst) {
  const ExpertLayout L = expert_layout(hidden, inter);
  pack_host(GateUpRows{gn, gs, un, us, inter}, L.gu, dst);
  pack_host(PlainRows{dn, ds, hidden}, L.down, dst + L.down_offset);
}

hipError_t launch_pack(const uint8_t *nib, const uint8_t *sc, int rows,
                       int cols, uint8_t *tiles, hipStream_t s) {
  const MatLayout m = mat_layout(rows, cols);
  const size_t n = (size_t)(5 * m.G4) * kTileRows * m.ntiles;
  hipLaunchKernelGGL(pack_kernel<PlainRows>, dim3(grid_for(n)), dim3(256), 0,
                     s, PlainRows{nib, sc, rows}, m, tiles);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *tiles, int rows, int cols,
                         uint8_t *nib, uint8_t *sc, hipStream_t s) {
  const MatLayout m = mat_layout(rows, cols);
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for((size_t)rows * m.G)),
                     dim3(256), 0, s, tiles, m, nib, sc);
  return hipGetLastError();
}

hipError_t launch_expert_pack(const uint8_t *gn, const uint8_t *gs,
                              const uint8_t *un, const uint8_t *us,
                              const uint8_t *dn, const uint8_t *ds, int hidden,
                              int inter, uint8_t *dst, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  size_t n = (size_t)(5 * L.gu.G4) * kTileRows * L.gu.ntiles;
  hipLaunchKernelGGL(pack_kernel<GateUpRows>, dim3(grid_for(n)), dim3(256), 0,
                     s, GateUpRows{gn, gs, un, us, inter}, L.gu, dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  n = (size_t)(5 * L.down.G4) * kTileRows * L.down.ntiles;
  hipLaunchKernelGGL(pack_kernel<PlainRows>, dim3(grid_for(n)), dim3(256), 0,
                     s, PlainRows{dn, ds, hidden}, L.down, dst + L.down_offset);
  return hipGetLastError();
}

}  // namespace k3
