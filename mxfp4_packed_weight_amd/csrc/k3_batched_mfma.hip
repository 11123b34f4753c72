// Batched decode on the matrix unit: each selected expert's gate/up and down
// tiles times the rows of its tokens, with v_mfma_f32_16x16x32_bf16.
//
// A decode batch gives an expert a few tokens, often only one, so this is
// still a stream of packed weight bytes; what the matrix unit removes is the
// per-token vector work. A vector kernel multiplies every decoded weight by
// every token on the vector ALU and fetches each token's activations with
// scalar loads, which stall it (one fetch per token per group). Here the
// weights are decoded once into a bf16 A operand, the tokens are the 16
// columns of B, and the activations reach the waves through LDS.
//
// Work: one workgroup of four waves per (work item of at most 16 tokens of one
// expert, four consecutive tiles); wave w computes C[64 rows][16 tokens] of
// one tile over the whole K. Its weights stream through its own ring of quads
// in LDS, filled by direct global -> LDS copies; per quad, wave w gathers
// group w of the quad for the item's 16 tokens into a shared LDS block, and
// after one barrier every wave reads all four blocks.
//
// Operands of one instruction (16 x 16 x 32 bf16): lane l holds row l%16 of A
// and column l%16 of B, K elements [8(l/16), +8) of both; C lane l holds
// column l%16, rows 4(l/16) + i. The K range of one instruction is one MXFP4
// group (32 codes), so a group's exponent applies to whole A rows: the codes
// are converted to bf16 with the group scale folded in (exact for exponent
// bytes 2..252: the largest code times 2^125 and the smallest nonzero one
// times 2^-125 are normal bf16). A quad that holds any other exponent byte
// (0, 1, 253, 254 or 255) in this wave's tile takes the exact route instead:
// each group's unscaled sum from its own instructions, then scaled into the
// accumulator with ldexp, as the vector kernels do. There a group with byte
// 255 is skipped, not multiplied by zero, so a NaN or infinite activation
// inside it does not reach the row ([A176] "What byte-identical actually
// costs").
//
// Gate/up multiplies bf16 x, which is exact in bf16. Down multiplies h, which
// is fp32: the gate/up epilogue writes it as three bf16 pieces whose sum is
// the fp32 value (hi = bf16(h), mid = bf16(h - hi), lo = h - hi - mid, each
// step exact), and down runs one instruction per piece. Products of bf16
// values are exact in fp32; the sums accumulate in fp32.
#include "k3_stream.h"

namespace k3 {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBmWaves = 4;   // tiles per workgroup, one per wave
constexpr int kBmTok = 16;    // tokens per work item: one column block
constexpr int kBmBDepth = 2;  // activation blocks in flight (registers)
constexpr int kPieces = 3;    // bf16 pieces of an fp32 h value

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kWaitLgkm0 = 0xC07F;
// Loads issued per quad: five weight copies (four of 16 bytes and one of 4
// per lane), then this wave's activation block (one 16-byte load per lane
// and piece).
constexpr int kBmLoadsA = 5;
template <int LB>
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case kBmLoadsA + LB: __builtin_amdgcn_s_waitcnt(vm_wait_imm(kBmLoadsA + LB)); break;
    case LB: __builtin_amdgcn_s_waitcnt(vm_wait_imm(LB)); break;
    case kBmLoadsA: __builtin_amdgcn_s_waitcnt(vm_wait_imm(kBmLoadsA)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_wait_imm(0)); break;
  }
}

// The three bf16 pieces of v (their fp32 sum is v; a non-finite v is all in
// the first piece). A finite v that rounds to a bf16 infinity (|v| within
// half a bf16 step of FLT_MAX) takes its first piece rounded toward zero
// instead, which keeps every piece finite and the residuals exact.
__device__ __forceinline__ void split3(float v, uint16_t &p0, uint16_t &p1, uint16_t &p2) {
  p0 = f32_to_bf16_rne(v);
  if (__builtin_isfinite(v) && (p0 & 0x7F80u) == 0x7F80u) p0 = (uint16_t)(__float_as_uint(v) >> 16);
  const float r1 = v - __uint_as_float((uint32_t)p0 << 16);
  p1 = f32_to_bf16_rne(r1);
  const float r2 = r1 - __uint_as_float((uint32_t)p1 << 16);
  p2 = f32_to_bf16_rne(r2);
  if (!__builtin_isfinite(v)) p1 = p2 = 0;
}

// Eight E2M1 codes (one dword: byte b holds codes 2b, 2b + 1, low nibble
// first) to eight bf16 values times `scale`, in code order.
__device__ __forceinline__ v8bf decode8(uint32_t w, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

struct BmItems {
  const int32_t *e, *off, *cnt, *n;
};

// kDown = false: gate/up. hp[piece][q][inter] = the bf16 pieces of
// SiLU(gate . x_tok) * (up . x_tok) for the pairs q of every work item, tok =
// pair_token[q]; tile rows 0..31 are gate rows, 32..63 the up rows of the
// same 32 outputs. kDown = true: yp[q][hidden] = W_down(e) h[q], h read as
// its pieces hp, by one of two launches: NP = 3 takes the items of more than
// kPackTok pairs (one instruction per piece); NP = 1 the others, whose
// (pair, piece) combinations fit the 16 columns of one instruction (column
// p * cnt + t holds piece p of pair t), the pieces' sums added at the end.
constexpr int kPackTok = 5;  // 3 * 5 <= 16 columns
template <bool kDown, int NP>
__global__ __launch_bounds__(kBmWaves * 64) void batched_mfma_kernel(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ pair_token,
    const uint8_t *const *__restrict__ experts, BmItems it, int hidden, int inter,
    long long P, uint16_t *__restrict__ hp, float *__restrict__ yp) {
  static_assert(NP == 1 || (kDown && NP == kPieces), "B pieces per instruction");
  constexpr bool kPacked = kDown && NP == 1;
  constexpr int kDepth = NP == 1 ? 2 : 3;  // weight quads in flight per wave
  constexpr int LB = NP;                               // activation loads per quad
  __shared__ u32x4 bl[kBmBDepth][NP][kBmWaves][64];    // B of one quad: group w, lane order
  __shared__ __attribute__((aligned(16))) uint8_t ring[kBmWaves][kDepth][kQuadBytes];
  const ExpertLayout L = expert_layout(hidden, inter);
  const MatLayout &M = kDown ? L.down : L.gu;
  const int Tt = M.ntiles, ngrp = (Tt + kBmWaves - 1) / kBmWaves;
  // this launch's items: gate/up all of them; down the first it.n[1] (more
  // than kPackTok pairs) for NP = 3, the others for NP = 1
  const int u = blockIdx.x;
  const int i_lo = kPacked ? ldc(it.n + 1) : 0, i_hi = kDown && !kPacked ? ldc(it.n + 1) : ldc(it.n);
  const int item = i_lo + u / ngrp;
  if (item >= i_hi) return;  // the whole workgroup leaves together
  const int wave = wave_id();
  const int s = kBmWaves * (u % ngrp) + wave;
  const bool active = s < Tt;  // else: streams tile Tt - 1, stores nothing
  const int e = ldc(it.e + item), off = ldc(it.off + item), cnt = ldc(it.cnt + item);
  if (kDown && (cnt <= kPackTok) != kPacked) return;  // not this launch's (never, when ordered)
  const uint8_t *tile = ldc(experts + e) + (kDown ? L.down_offset : 0) +
                        (size_t)(active ? s : Tt - 1) * M.tile_bytes;
  const int G = M.G, G4 = M.G4;
  const int lane = threadIdx.x & 63, col = lane & 15, kb = lane >> 4;
  // the activation row of this lane's column (a column past the item reads
  // the item's first row; its results are never stored): x of its token, or
  // the first piece of its pair's h (piece p is p * P rows further); packed:
  // column p * cnt + t is piece p of pair t
  const size_t pstride = (size_t)P * inter;
  const uint16_t *brow;
  if constexpr (kPacked) {
    const bool used = col < kPieces * cnt;
    const int t = used ? col % cnt : 0, pc = used ? col / cnt : 0;
    brow = hp + pc * pstride + (size_t)(off + t) * inter;
  } else {
    const int c = off + (col < cnt ? col : 0);
    brow = kDown ? hp + (size_t)c * inter : X + (size_t)pair_token[c] * hidden;
  }

  u32x4 b[kBmBDepth][NP];
  auto load_a = [&](int slot, int q) __attribute__((always_inline)) {
    const uint8_t *qb = tile + (size_t)kQuadBytes * q;
    uint8_t *dst = ring[wave][slot];
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the slot's last reads are done
    asm volatile("" ::: "memory");
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(qb + 1024 * c4 + 16 * lane),
                                       (lvoid_t *)(dst + 1024 * c4), 16, 0, 2);
    __builtin_amdgcn_global_load_lds((gvoid_t *)(qb + 4096 + 4 * lane),
                                     (lvoid_t *)(dst + 4096), 4, 0, 2);
  };
  auto load_b = [&](int d, int q) __attribute__((always_inline)) {
    const int g = min(4 * q + wave, G - 1);  // groups past G are skipped
#pragma unroll
    for (int p = 0; p < NP; ++p)
      b[d][p] = *(const gu4_t *)(brow + p * pstride + 32 * g + 8 * kb);
  };
  v4f acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int slot, int d, int q) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p) bl[d][p][wave][lane] = b[d][p];
    // barrier without a fence (a fence would also wait for the weight copies
    // in flight and drain the ring at every quad)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    v8bf bv[NP][4];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int g = 0; g < 4; ++g) bv[p][g] = __builtin_bit_cast(v8bf, bl[d][p][g][lane]);
    // A words: row 16m + col, group g, codes [8kb, +8) at ring offset
    // 1024g + 16(16m + col) + 4kb = base + 256(4g + m); the row's exponent
    // word (its four groups' bytes) at 4096 + 4(16m + col). One block that
    // waits for its own reads: the copies are known complete from the
    // explicit vmcnt wait before this step.
    u32x2 aw[8];
    uint32_t sr[4];
    typedef __attribute__((address_space(3))) const uint8_t lds_u8;
    const uint32_t qa = (uint32_t)(size_t)(lds_u8 *)ring[wave][slot];
    {
      const uint32_t va = qa + 16 * col + 4 * kb, vs = qa + 4096 + 4 * col;
      asm volatile(
          "ds_read2st64_b32 %0, %12 offset0:0 offset1:4\n"
          "ds_read2st64_b32 %1, %12 offset0:8 offset1:12\n"
          "ds_read2st64_b32 %2, %12 offset0:1 offset1:5\n"
          "ds_read2st64_b32 %3, %12 offset0:9 offset1:13\n"
          "ds_read2st64_b32 %4, %12 offset0:2 offset1:6\n"
          "ds_read2st64_b32 %5, %12 offset0:10 offset1:14\n"
          "ds_read2st64_b32 %6, %12 offset0:3 offset1:7\n"
          "ds_read2st64_b32 %7, %12 offset0:11 offset1:15\n"
          "ds_read_b32 %8, %13\n"
          "ds_read_b32 %9, %13 offset:64\n"
          "ds_read_b32 %10, %13 offset:128\n"
          "ds_read_b32 %11, %13 offset:192\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(aw[0]), "=&v"(aw[1]), "=&v"(aw[2]), "=&v"(aw[3]), "=&v"(aw[4]),
            "=&v"(aw[5]), "=&v"(aw[6]), "=&v"(aw[7]), "=&v"(sr[0]), "=&v"(sr[1]),
            "=&v"(sr[2]), "=&v"(sr[3])
          : "v"(va), "v"(vs)
          : "memory");
    }
    // word of (m, g): aw[2m + g/2][g%2]
    bool odd = false;  // an exponent byte the folded scale cannot take, or 255
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t ex = (sr[m] >> (8 * g)) & 255u;
        odd |= ex - 2u > 250u;
      }
    if (__ballot(odd) == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (4 * q + g < G) {  // wave-uniform
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t ex = (sr[m] >> (8 * g)) & 255u;  // 2..252 here
            const v8bf a = decode8(aw[2 * m + g / 2][g % 2], __uint_as_float(ex << 23));
#pragma unroll
            for (int p = 0; p < NP; ++p)
              acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv[p][g], acc[m], 0, 0, 0);
          }
        }
      }
    } else {
      // exponents of this lane's C rows 16m + 4kb + i (a word per row)
      u32x4 ec[4];
      asm volatile(
          "ds_read_b128 %0, %4\n"
          "ds_read_b128 %1, %4 offset:64\n"
          "ds_read_b128 %2, %4 offset:128\n"
          "ds_read_b128 %3, %4 offset:192\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(ec[0]), "=&v"(ec[1]), "=&v"(ec[2]), "=&v"(ec[3])
          : "v"(qa + 4096 + 16 * kb)
          : "memory");
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (4 * q + g < G) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const v8bf a = decode8(aw[2 * m + g / 2][g % 2], 1.0f);
            v4f part = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NP; ++p)
              part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv[p][g], part, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[m][i] = apply_scale(acc[m][i], part[i], (ec[m][i] >> (8 * g)) & 255u);
          }
        }
      }
    }
  };
  // Loads issued after quad q's activation block (its last loads) by the
  // time quad q is consumed: quad 0's block is followed by quad 1's; quad
  // q >= 1's by step q - 1's weights (quad q - 1 + kDepth) and block (quad
  // q - 1 + kBmBDepth), when those exist.
  auto after = [&](int q) __attribute__((always_inline)) {
    if (q == 0) return G4 > 1 ? LB : 0;
    return (q - 1 + kDepth < G4 ? kBmLoadsA : 0) + (q - 1 + kBmBDepth < G4 ? LB : 0);
  };
  auto steady = [&](int q, int d) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(kBmLoadsA + LB));  // quad q is in
    asm volatile("" ::: "memory");
    consume(q % kDepth, d, q);
    load_a(q % kDepth, q + kDepth);
    load_b(d, q + kBmBDepth);
  };
  auto tail = [&](int q, int d) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    wait_vmcnt<LB>(after(q));
    asm volatile("" ::: "memory");
    consume(q % kDepth, d, q);
    if (q + kDepth < G4) load_a(q % kDepth, q + kDepth);
    if (q + kBmBDepth < G4) load_b(d, q + kBmBDepth);
  };
  if (G4 >= kDepth + 2) {
#pragma unroll
    for (int q = 0; q < kDepth; ++q) load_a(q, q);
    load_b(0, 0);
    load_b(1, 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(LB));  // quad 0 is in
    asm volatile("" ::: "memory");
    consume(0, 0, 0);
    load_a(0, kDepth);
    load_b(0, kBmBDepth);
    int q = 1;
    for (; q + 1 + kDepth < G4; q += 2) {
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
    for (int q = 0; q < min(kDepth, G4); ++q) load_a(q, q);
    load_b(0, 0);
    if (G4 > 1) load_b(1, 1);
    for (int q = 0; q < G4; ++q) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
      asm volatile("" ::: "memory");
      if (q & 1) {
        consume(q % kDepth, 1, q);
        if (q + kDepth < G4) load_a(q % kDepth, q + kDepth);
        if (q + kBmBDepth < G4) load_b(1, q + kBmBDepth);
      } else {
        consume(q % kDepth, 0, q);
        if (q + kDepth < G4) load_a(q % kDepth, q + kDepth);
        if (q + kBmBDepth < G4) load_b(0, q + kBmBDepth);
      }
    }
  }

  if constexpr (kPacked) {  // column t += columns cnt + t and 2 cnt + t (same lane group)
    const int src1 = min(lane + cnt, 63), src2 = min(lane + 2 * cnt, 63);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v1 = __shfl(acc[m][i], src1), v2 = __shfl(acc[m][i], src2);
        acc[m][i] = (acc[m][i] + v1) + v2;
      }
  }
  if (!active || col >= cnt) return;  // padding wave, or a column past the item
  const size_t q = (size_t)(off + col);
  if constexpr (kDown) {
    // C rows 16m + 4kb + i of tile s (hidden % 32 == 0: a group of four
    // rows is wholly in or out)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 64 * s + 16 * m + 4 * kb;
      if (row < hidden)  // non-temporal: read once, by the combine
        __builtin_nontemporal_store(acc[m], reinterpret_cast<v4f *>(yp + q * hidden + row));
    }
  } else {
    // C rows 16m + 4kb + i: m = 0, 1 gate rows, m = 2, 3 the up rows of the
    // same outputs 32s + 16m + 4kb + i (inter % 32 == 0: all exist)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const v4f g = acc[m], up = acc[m + 2];
      uint16_t pc[kPieces][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split3(silu(g[i]) * up[i], pc[0][i], pc[1][i], pc[2][i]);
      const size_t at = q * inter + 32 * s + 16 * m + 4 * kb;
#pragma unroll
      for (int p = 0; p < kPieces; ++p)
        *reinterpret_cast<uint2 *>(hp + p * pstride + at) =
            uint2{pc[p][0] | ((uint32_t)pc[p][1] << 16), pc[p][2] | ((uint32_t)pc[p][3] << 16)};
    }
  }
}

}  // namespace

int gate_up_mfma_tok() { return kBmTok; }
int down_mfma_pack_tok() { return kPackTok; }

// max_items: an upper bound of the work items the permutation can make.
hipError_t launch_gate_up_mfma(const uint16_t *X, const uint8_t *const *experts,
                               const PermOut &o, int max_items, long long P, int hidden,
                               int inter, uint16_t *hp, hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const BmItems it{o.item_e, o.item_off, o.item_cnt, o.n_items};
  const long long ngrp = (L.gu.ntiles + kBmWaves - 1) / kBmWaves;
  hipLaunchKernelGGL((batched_mfma_kernel<false, 1>), dim3((unsigned)(max_items * ngrp)),
                     dim3(kBmWaves * 64), 0, s, X, o.pair_token, experts, it, hidden, inter, P,
                     hp, nullptr);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const uint16_t *hp, const uint8_t *const *experts, const PermOut &o,
                            int max_items, long long P, int hidden, int inter, float *yp,
                            hipStream_t s) {
  const ExpertLayout L = expert_layout(hidden, inter);
  const BmItems it{o.item_e, o.item_off, o.item_cnt, o.n_items};
  const long long ngrp = (L.down.ntiles + kBmWaves - 1) / kBmWaves;
  // the items of at most kPackTok pairs (after the others in the item
  // order), then the others
  hipLaunchKernelGGL((batched_mfma_kernel<true, 1>), dim3((unsigned)(max_items * ngrp)),
                     dim3(kBmWaves * 64), 0, s, nullptr, o.pair_token, experts, it, hidden, inter,
                     P, const_cast<uint16_t *>(hp), yp);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the first class holds at most P / (kPackTok + 1) items
  const long long n_large = std::min<long long>(max_items, P / (kPackTok + 1));
  if (n_large < 1) return hipSuccess;
  hipLaunchKernelGGL((batched_mfma_kernel<true, kPieces>), dim3((unsigned)(n_large * ngrp)),
                     dim3(kBmWaves * 64), 0, s, nullptr, o.pair_token, experts, it, hidden, inter,
                     P, const_cast<uint16_t *>(hp), yp);
  return hipGetLastError();
}

}  // namespace k3
