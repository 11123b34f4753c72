/*
 * k3gen — seeded synthetic inputs for the MXFP4 routed-expert path.
 *
 * This module is test and benchmark infrastructure shared by the oracle side
 * and the GPU side. It only draws random numbers and lays them out as the
 * canonical tensors both sides consume; it contains none of the arithmetic of
 * the method itself (no decode, no product, no routing, no combine).
 *
 * Random numbers come from SplitMix64 used as a counter-based generator: the
 * i-th value of stream `key` is the (i+1)-th output of a SplitMix64 sequence
 * whose state starts at `key` (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). Any element of any tensor can
 * be regenerated alone, so e.g. one expert of a 896-expert pool is produced
 * without the others.
 *
 * Canonical MXFP4 layout produced here (the layout the oracle reads):
 *   nib[r][K/2]  byte b of row r holds elements 2b (low nibble) and 2b+1
 *                (high nibble);
 *   sc[r][K/32]  one E8M0 exponent byte per 32 consecutive elements of a row.
 */
#ifndef K3GEN_H
#define K3GEN_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tensor kinds used to derive independent stream keys. */
enum {
  K3G_KIND_MATRIX = 1, /* one standalone MXFP4 matrix            */
  K3G_KIND_EXPERT = 2, /* routed expert weights (gate, up, down)  */
  K3G_KIND_ROUTER = 3, /* bf16 router weight                      */
  K3G_KIND_TOKENS = 4, /* activations                             */
  K3G_KIND_LOGITS = 5, /* synthetic router logits                 */
  K3G_KIND_BIAS = 6,   /* routing bias                            */
  K3G_KIND_PERM = 7    /* expert popularity permutation           */
};

/* SplitMix64 output function applied to state s (one "next" step's mix). */
uint64_t k3g_mix64(uint64_t s);
/* Classic sequential SplitMix64: advances *state by the golden gamma and
 * returns the mixed value. */
uint64_t k3g_splitmix64_next(uint64_t *state);
/* Counter-based access: value i (i >= 0) of the stream started at `key`,
 * identical to the (i+1)-th call of k3g_splitmix64_next from state key. */
uint64_t k3g_draw(uint64_t key, uint64_t i);
/* Stream key for (seed, config, kind, a, b). */
uint64_t k3g_key(uint64_t seed, uint32_t cfg, uint32_t kind, uint32_t a,
                 uint32_t b);

/* out[i] = byte (i % 8) (little-endian) of draw(key, i / 8). */
void k3g_bytes(uint64_t key, uint8_t *out, size_t n);
/* out[i] = lo + floor(((draw(key,i) >> 32) * (hi - lo + 1)) / 2^32). */
void k3g_uniform_u8(uint64_t key, int lo, int hi, uint8_t *out, size_t n);
/* Standard normal pairs by Box-Muller in fp64 from draws 2j, 2j+1, then
 * mu + sigma*z rounded to fp32 (round-to-nearest-even). */
void k3g_normal_f32(uint64_t key, double mu, double sigma, float *out,
                    size_t n);
/* As k3g_normal_f32, then the fp32 value rounded to bf16 (RNE). */
void k3g_normal_bf16(uint64_t key, double mu, double sigma, uint16_t *out,
                     size_t n);
/* fp32 in [0,1): top 24 bits of each draw times 2^-24 (exact). */
void k3g_uniform_f32(uint64_t key, float *out, size_t n);
/* fp32 round-to-nearest-even to bf16 bits (NaN kept quiet). */
uint16_t k3g_f32_to_bf16(float f);

/* One canonical MXFP4 matrix: codes uniform over 16 (every nibble), exponent
 * bytes uniform in [elo, ehi]. Keys: (seed,cfg,kind,a,2b) for codes and
 * (seed,cfg,kind,a,2b+1) for exponents. */
void k3g_mxfp4_matrix(uint64_t seed, uint32_t cfg, uint32_t kind, uint32_t a,
                      uint32_t b, int rows, int cols, int elo, int ehi,
                      uint8_t *nib, uint8_t *sc);

/* One routed expert: gate[inter][hidden], up[inter][hidden],
 * down[hidden][inter]; matrix ids 0, 1, 2 under kind K3G_KIND_EXPERT and
 * a = expert id. Any pointer may be NULL to skip that matrix. */
void k3g_expert(uint64_t seed, uint32_t cfg, uint32_t expert, int hidden,
                int inter, int elo, int ehi, uint8_t *gate_nib,
                uint8_t *gate_sc, uint8_t *up_nib, uint8_t *up_sc,
                uint8_t *down_nib, uint8_t *down_sc);

/* Zipf-skewed router logits: l[t][e] = ln p(rank(e)) + Gumbel(0,1), where
 * p(r) ~ r^-s over ranks 1..n and rank(e) is a seeded permutation of the
 * experts (Fisher-Yates driven by the PERM stream, fixed per seed); the
 * Gumbel noise is drawn per `batch`. Rounded to fp32. Top-k of such logits
 * is a draw without replacement with probabilities p. */
void k3g_zipf_logits(uint64_t seed, uint32_t cfg, uint32_t batch, int T, int n,
                     double s, float *out);

/* Number of threads the bulk generators may use (default: 1). */
void k3g_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
