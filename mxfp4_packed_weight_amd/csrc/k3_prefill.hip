// Prefill: the grouped GEMMs of many tokens per expert on gfx950's
// block-scaled FP4 matrix instruction, v_mfma_scale_f32_16x16x128_f8f6f4
// with both operands FP4 (E2M1 codes and per-32 E8M0 exponents). This is
// the path's one dense contraction: every expert sees tens of tokens, so
// its packed weights are multiplied as a matrix, not a vector.
//
// Activations are quantised to MXFP4 per 32 along K (x before gate/up, h
// before down) by the rule of the oracle's quantiser: E = floor(log2 amax)
// - 2 clamped to [-127, 127], codes = E2M1 nearest to v / 2^E with ties to
// the even code, saturating at 6; an all-zero block has exponent 0.
//
// Operand layouts of the instruction (16 x 16 x 128, both FP4; measured):
//   A: lane l = row l%16, K elements [32(l/16), +32): 16 bytes, low nibble
//      even, which is exactly one MXFP4 group of one weight row; its scale
//      is that group's exponent byte.
//   B: lane l = column l%16, the same K range of that column: one group of
//      one token's quantised row, with that group's exponent as its scale.
//   C: lane l = column l%16, rows 4(l/16) + i, i = 0..3.
// Every product of two E2M1 values times two powers of two is exact, and
// within a 32-block they span less than 2^8, below the unit's alignment
// window, so the block sums are exact and accumulate in fp32.
#include "k3_stream.h"

namespace k3 {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kNB = 4;                 // 16-token column blocks per work item
constexpr int kPfTok = 16 * kNB;       // tokens per prefill work item
#ifndef K3_PF_DEPTH
#define K3_PF_DEPTH 2
#endif
constexpr int kPfDepth = K3_PF_DEPTH;  // weight quads in flight per wave (LDS)
constexpr int kPfBDepth = 2;           // activation quads in flight (registers)
constexpr int kPfWaves = kNB;          // weight tiles (waves) per workgroup

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// s_waitcnt immediates: vmcnt(n) with the other counters left free, and
// lgkmcnt(0) with vmcnt and expcnt left free.
constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kWaitLgkm0 = 0xC07F;
// Loads issued per quad: five weight copies (four of 16 bytes and one of 4
// per lane), then this wave's activation block (16 bytes and one byte).
constexpr int kPfLoadsA = 5, kPfLoadsB = 2;
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case kPfLoadsA + kPfLoadsB: __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPfLoadsA + kPfLoadsB)); break;
    case kPfLoadsB: __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPfLoadsB)); break;
    case kPfLoadsA: __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPfLoadsA)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_wait_imm(0)); break;
  }
}

// |v| / 2^E (exact) -> E2M1 magnitude code, nearest with ties to the even
// code (0, 1.0, 2.0, 4.0), saturating at 6.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  if (a <= 0.25f) return 0u;
  if (a < 0.75f) return 1u;
  if (a <= 1.25f) return 2u;
  if (a < 1.75f) return 3u;
  if (a <= 2.5f) return 4u;
  if (a < 3.5f) return 5u;
  if (a <= 5.0f) return 6u;
  return 7u;
}

// Exponent byte of a block with largest magnitude amax, and 2^-E.
__device__ __forceinline__ uint32_t mx_scale(float amax, float *inv) {
  if (!(amax > 0.f)) {
    *inv = 0.f;
    return 0u;
  }
  const int ef = (int)((__float_as_uint(amax) >> 23) & 255u);
  const int E = max(-127, (ef == 0 ? -127 : ef - 127) - 2);
  *inv = __uint_as_float((uint32_t)(127 - E) << 23);
  return (uint32_t)(E + 127);
}

// E2M1 code of v under 2^-E (sign kept only for a nonzero magnitude).
__device__ __forceinline__ uint32_t e2m1_code(float v, float inv) {
  const uint32_t m = e2m1_mag_code(fabsf(v) * inv);
  return (m != 0u && v < 0.f) ? (m | 8u) : m;
}

// Quantiser: v[rows][cols] -> nib[rows][cols/2] (element 2b in the low
// nibble of byte b) and sc[rows][cols/32]. One lane per block of 32 values:
// 16-byte loads of the block, its largest magnitude, the block exponent and
// 32 codes (each by the same rule), one 16-byte store of the codes and one
// exponent byte. Rows are a multiple of 32 values, and v and nib are 16-byte
// aligned (the ABI refuses other buffers).
template <typename T>
__global__ __launch_bounds__(256) void quant_kernel(const T *__restrict__ v,
                                                    long long nblocks, int cols,
                                                    uint8_t *__restrict__ nib,
                                                    uint8_t *__restrict__ sc) {
  const long long blk = (long long)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  const int G = cols / 32;
  const long long r = blk / G, g = blk % G;
  float x[32];
  if constexpr (sizeof(T) == 2) {
    const uint4 *src = reinterpret_cast<const uint4 *>(v + r * cols + g * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = src[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
        x[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  } else {
    const float4 *src = reinterpret_cast<const float4 *>(v + r * cols + g * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 f = src[q];
      x[4 * q] = f.x;
      x[4 * q + 1] = f.y;
      x[4 * q + 2] = f.z;
      x[4 * q + 3] = f.w;
    }
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(x[i]));
  float inv;
  const uint32_t e = mx_scale(a, &inv);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i / 8] |= e2m1_code(x[i], inv) << (4 * (i % 8));
  *reinterpret_cast<uint4 *>(nib + r * (cols / 2) + g * 16) = uint4{w[0], w[1], w[2], w[3]};
  sc[r * G + g] = (uint8_t)e;
}

struct PfItems {
  const int32_t *e, *off, *cnt, *n;
};

// One workgroup of kPfWaves waves per (work item, group of kPfWaves
// consecutive weight tiles); wave w computes C[64 rows][up to 64 tokens] of
// tile s = kPfWaves * group + w over the whole K of the matrix. kGateUp: the
// gate/up stack (A = tile s of the expert's gate/up region, B = quantised x
// rows of the item's tokens); epilogue h = SiLU(gate) * up, quantised per 32
// (one group per tile) into hq[pair]; optional fp32 h. Otherwise the down
// matrix (B = quantised h rows of the item's pairs); epilogue yp[pair][row]
// fp32.
//
// The waves of a workgroup share the item's activations: per quad, wave w
// gathers only column block w of B (16 tokens x 4 groups, 16 bytes and one
// exponent byte per lane) and writes it to a double-buffered LDS slot; after
// one barrier every wave reads all four blocks from LDS. The gathers touch
// 16 cache lines per instruction, and sharing them cuts their number per
// wave by four. The weights stream through each wave's own ring of quads in
// LDS (below).
template <bool kGateUp>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_gemm_kernel(
    const uint8_t *__restrict__ bq, const uint8_t *__restrict__ bsc,
    const int32_t *__restrict__ pair_token, const uint8_t *const *__restrict__ experts,
    PfItems it, int hidden, int inter, uint8_t *__restrict__ hq,
    uint8_t *__restrict__ hsc, float *__restrict__ h32, float *__restrict__ yp) {
  static_assert(kPfWaves == kNB, "wave w gathers column block w");
  __shared__ u32x4 bl[kPfBDepth][kNB][64];     // B codes of a quad, lane order
  __shared__ uint8_t bsl[kPfBDepth][kNB][64];   // their exponent bytes
  const ExpertLayout L = expert_layout(hidden, inter);
  const MatLayout &M = kGateUp ? L.gu : L.down;
  const int Tt = M.ntiles, ngrp = (Tt + kPfWaves - 1) / kPfWaves;
  const int u = xcd_unit(blockIdx.x, ngrp);
  if (u >= ldc(it.n) * ngrp) return;  // the whole workgroup leaves together
  const int wave = wave_id();
  const int item = u / ngrp, s = kPfWaves * (u % ngrp) + wave;
  const bool active = s < Tt;  // else: streams tile Tt - 1, stores nothing
  const int e = ldc(it.e + item), off = ldc(it.off + item), cnt = ldc(it.cnt + item);
  const uint8_t *tile = ldc(experts + e) + (kGateUp ? 0 : L.down_offset) +
                        (size_t)(active ? s : Tt - 1) * M.tile_bytes;
  const int K = M.cols, G = M.G, G4 = M.G4;
  const int lane = threadIdx.x & 63, col = lane & 15, kb = lane >> 4;

  // which columns of each block hold tokens; the B row this lane gathers
  // for its wave's own block (clamped to a valid row)
  bool bok[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) bok[nb] = 16 * nb + col < cnt;
  const uint8_t *brow, *bsrow;
  {
    const int c = 16 * wave + col;
    const int q = off + (c < cnt ? c : 0);
    const long long r = kGateUp ? (long long)ldc(pair_token + q) : (long long)q;
    brow = bq + r * (K / 2);
    bsrow = bsc + r * G;
  }

  // Weights: a ring of kPfDepth quads per wave in LDS, each slot a verbatim
  // copy of one 4352-byte quad written by direct global -> LDS loads
  // (non-temporal: each weight byte is read once), so no register holds
  // weight bytes in flight. The compiler's own waits around such copies are
  // missing or too conservative (vmcnt(0)), so a slot is read only after an
  // explicit vmcnt wait derived from the issue order, by reads it does not
  // see (one asm block, below), and refilled only after those completed.
  __shared__ __attribute__((aligned(16))) uint8_t ring[kPfWaves][kPfDepth][kQuadBytes];
  u32x4 b[kPfBDepth];
  uint8_t bs[kPfBDepth];  // widened only where used (no early wait for it)
  auto load_a = [&](int slot, int q) {
    const uint8_t *qb = tile + (size_t)kQuadBytes * q;
    uint8_t *dst = ring[wave][slot];
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the slot's last reads are done
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < 4; ++c)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(qb + 1024 * c + 16 * lane),
                                       (lvoid_t *)(dst + 1024 * c), 16, 0, 2);
    __builtin_amdgcn_global_load_lds((gvoid_t *)(qb + 4096 + 4 * lane),
                                     (lvoid_t *)(dst + 4096), 4, 0, 2);
  };
  auto load_b = [&](int d, int q) {
    const int g = min(4 * q + kb, G - 1);  // groups past G are zero below
    b[d] = *(const gu4_t *)(brow + 16 * g);
    bs[d] = *(__attribute__((address_space(1))) const uint8_t *)(bsrow + g);
  };
  v4f acc[kNB][4];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[nb][m] = v4f{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int slot, int d, int q) {
    // share this wave's block of quad q; slot d was last read two quads ago,
    // before the previous barrier. The exponent byte stays a byte until it is
    // read back, so that nothing widens it (and waits for its load) early.
    bl[d][wave][lane] = b[d];
    bsl[d][wave][lane] = bs[d];
    // Barrier without a fence: the blocks are plain LDS writes, complete
    // after lgkmcnt(0). (A fence would also wait for the weight copies in
    // flight, vmcnt(0), and drain the ring at every quad.)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const bool gin = 4 * q + kb < G;
    // B operands once per quad: a column past the item or a group past K
    // contributes nothing (zero codes, unit scale)
    v8i bv[kNB];
    int eb[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const bool use = bok[nb] && gin;
      const u32x4 bm = bl[d][nb][lane];
      bv[nb] = v8i{use ? (int)bm.x : 0, use ? (int)bm.y : 0, use ? (int)bm.z : 0,
                   use ? (int)bm.w : 0, 0, 0, 0, 0};
      eb[nb] = use ? (int)bsl[d][nb][lane] : 127;
    }
    // This lane's A operands of the quad: the codes of rows 16m + col of
    // group 4q + kb and their exponent words, m = 0..3. Read in one block
    // that waits for its own reads: the slot's copy is known complete from
    // the explicit vmcnt wait before this step, and reads the compiler does
    // not see get no conservative vmcnt(0) of its own.
    u32x4 ar[4];
    uint32_t sr[4];
    {
      typedef __attribute__((address_space(3))) const uint8_t lds_u8;
      const uint32_t qa = (uint32_t)(size_t)(lds_u8 *)ring[wave][slot];
      const uint32_t va = qa + 1024 * kb + 16 * col, vs = qa + 4096 + 4 * col;
      asm volatile(
          "ds_read_b128 %0, %8\n"
          "ds_read_b128 %1, %8 offset:256\n"
          "ds_read_b128 %2, %8 offset:512\n"
          "ds_read_b128 %3, %8 offset:768\n"
          "ds_read_b32 %4, %9\n"
          "ds_read_b32 %5, %9 offset:64\n"
          "ds_read_b32 %6, %9 offset:128\n"
          "ds_read_b32 %7, %9 offset:192\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(ar[0]), "=&v"(ar[1]), "=&v"(ar[2]), "=&v"(ar[3]), "=&v"(sr[0]),
            "=&v"(sr[1]), "=&v"(sr[2]), "=&v"(sr[3])
          : "v"(va), "v"(vs)
          : "memory");
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u32x4 am = ar[m];
      uint32_t ea = (sr[m] >> (8 * kb)) & 255u;
      if (ea == 255u) {  // the group contributes nothing
        am = u32x4{0u, 0u, 0u, 0u};
        ea = 127u;
      }
      const v8i av = {(int)am.x, (int)am.y, (int)am.z, (int)am.w, 0, 0, 0, 0};
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        acc[nb][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av, bv[nb], acc[nb][m], 4, 4, 0, (int)ea, 0, eb[nb]);
    }
  };
  // Loads issued after quad q's activation block (the last loads of quad q)
  // when quad q is consumed: quad 0's block is followed by quad 1's; quad
  // q >= 1's by step q - 1's weights (quad q - 1 + kPfDepth) and block
  // (quad q - 1 + kPfBDepth), when those exist.
  auto after = [&](int q) {
    if (q == 0) return G4 > 1 ? kPfLoadsB : 0;
    return (q - 1 + kPfDepth < G4 ? kPfLoadsA : 0) + (q - 1 + kPfBDepth < G4 ? kPfLoadsB : 0);
  };
  // a step whose next loads both exist: unconditional loads and a constant
  // wait keep the compiler's own waits exact (no register merges)
  auto steady = [&](int q, int d) {
    asm volatile("" ::: "memory");  // no earlier load sinks below the wait
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPfLoadsA + kPfLoadsB));  // quad q is in
    asm volatile("" ::: "memory");
    consume(q % kPfDepth, d, q);
    load_a(q % kPfDepth, q + kPfDepth);
    load_b(d, q + kPfBDepth);
  };
  auto tail = [&](int q, int d) {
    asm volatile("" ::: "memory");
    wait_vmcnt(after(q));
    asm volatile("" ::: "memory");
    consume(q % kPfDepth, d, q);
    if (q + kPfDepth < G4) load_a(q % kPfDepth, q + kPfDepth);
    if (q + kPfBDepth < G4) load_b(d, q + kPfBDepth);
  };
  if (G4 >= kPfDepth + 2) {
#pragma unroll
    for (int q = 0; q < kPfDepth; ++q) load_a(q, q);
    load_b(0, 0);
    load_b(1, 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPfLoadsB));  // quad 0 is in
    asm volatile("" ::: "memory");
    consume(0, 0, 0);
    load_a(0, kPfDepth);
    load_b(0, kPfBDepth);
    int q = 1;
    for (; q + 1 + kPfDepth < G4; q += 2) {
      steady(q, 1);
      steady(q + 1, 0);
    }
    for (; q < G4; ++q) {
      if (q & 1)
        tail(q, 1);
      else
        tail(q, 0);
    }
  } else {  // short K: every step waits for all of its loads
    for (int q = 0; q < min(kPfDepth, G4); ++q) load_a(q, q);
    load_b(0, 0);
    if (G4 > 1) load_b(1, 1);
    for (int q = 0; q < G4; ++q) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
      asm volatile("" ::: "memory");
      if (q & 1) {
        consume(q % kPfDepth, 1, q);
        if (q + kPfDepth < G4) load_a(q % kPfDepth, q + kPfDepth);
        if (q + kPfBDepth < G4) load_b(1, q + kPfBDepth);
      } else {
        consume(q % kPfDepth, 0, q);
        if (q + kPfDepth < G4) load_a(q % kPfDepth, q + kPfDepth);
        if (q + kPfBDepth < G4) load_b(0, q + kPfBDepth);
      }
    }
  }

  if (!active) return;  // a padding wave of a ragged tile group
  const int j = lane >> 4;  // C rows 4j + i of each 16-row sub-block
  if constexpr (kGateUp) {
    // tile rows 0..31 gate, 32..63 up (the same 32 output rows 32s + r)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      float hv[2][4];
      float amax = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hv[m][i] = silu(acc[nb][m][i]) * acc[nb][m + 2][i];
          amax = fmaxf(amax, fabsf(hv[m][i]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      if (!bok[nb]) continue;
      const size_t p = (size_t)off + 16 * nb + col;
      float inv;
      const uint32_t ex = mx_scale(amax, &inv);
      // rows r = 16m + 4j + i: bytes (16m + 4j)/2 and +1 of the group
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t c0 = e2m1_code(hv[m][0], inv), c1 = e2m1_code(hv[m][1], inv);
        const uint32_t c2 = e2m1_code(hv[m][2], inv), c3 = e2m1_code(hv[m][3], inv);
        uint8_t *dst = hq + p * (inter / 2) + (size_t)16 * s + 8 * m + 2 * j;
        dst[0] = (uint8_t)(c0 | (c1 << 4));
        dst[1] = (uint8_t)(c2 | (c3 << 4));
        if (h32) {
          float *hd = h32 + p * inter + (size_t)32 * s + 16 * m + 4 * j;
          *reinterpret_cast<v4f *>(hd) = v4f{hv[m][0], hv[m][1], hv[m][2], hv[m][3]};
        }
      }
      if (j == 0) hsc[p * (inter / 32) + s] = (uint8_t)ex;
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      if (!bok[nb]) continue;
      const size_t p = (size_t)off + 16 * nb + col;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 64 * s + 16 * m + 4 * j;
        if (row < hidden)  // non-temporal: read once, by the combine
          __builtin_nontemporal_store(acc[nb][m], reinterpret_cast<v4f *>(yp + p * hidden + row));
      }
    }
  }
}

}  // namespace

int prefill_tok_batch() { return kPfTok; }

hipError_t launch_quant_bf16(const uint16_t *v, long long rows, int cols,
                             uint8_t *nib, uint8_t *sc, hipStream_t s) {
  const long long nblocks = rows * (cols / 32);
  hipLaunchKernelGGL(quant_kernel<uint16_t>, dim3((unsigned)((nblocks + 255) / 256)),
                     dim3(256), 0, s, v, nblocks, cols, nib, sc);
  return hipGetLastError();
}

hipError_t launch_quant_f32(const float *v, long long rows, int cols,
                            uint8_t *nib, uint8_t *sc, hipStream_t s) {
  const long long nblocks = rows * (cols / 32);
  hipLaunchKernelGGL(quant_kernel<float>, dim3((unsigned)((nblocks + 255) / 256)),
                     dim3(256), 0, s, v, nblocks, cols, nib, sc);
  return hipGetLastError();
}

// max_items: an upper bound of the work items the permutation can make.
hipError_t launch_prefill_gate_up(const uint8_t *xq, const uint8_t *xsc,
                                  const uint8_t *const *experts,
                                  const PermOut &o, int max_items, int hidden,
                                  int inter, uint8_t *hq, uint8_t *hsc,
                                  float *h32, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const PfItems it{o.item_e, o.item_off, o.item_cnt, o.n_items};
  const long long ngrp = (L.gu.ntiles + kPfWaves - 1) / kPfWaves;
  hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3((unsigned)xcd_grid(max_items, ngrp)),
                     dim3(kPfWaves * 64),
                     0, s, xq, xsc, o.pair_token, experts, it, hidden, inter, hq,
                     hsc, h32, nullptr);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const uint8_t *hq, const uint8_t *hsc,
                               const uint8_t *const *experts, const PermOut &o,
                               int max_items, int hidden, int inter, float *yp,
                               hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const PfItems it{o.item_e, o.item_off, o.item_cnt, o.n_items};
  const long long ngrp = (L.down.ntiles + kPfWaves - 1) / kPfWaves;
  hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3((unsigned)xcd_grid(max_items, ngrp)),
                     dim3(kPfWaves * 64), 0, s, hq, hsc, o.pair_token, experts, it, hidden,
                     inter, nullptr, nullptr, nullptr, yp);
  return hipGetLastError();
}

}  // namespace k3
