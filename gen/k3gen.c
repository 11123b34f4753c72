/*
 * k3gen — seeded synthetic inputs (see k3gen.h). Plain C99 + optional OpenMP.
 * Only random draws and data layout live here; none of the method's
 * arithmetic does.
 */
#include "k3gen.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define K3G_GAMMA 0x9E3779B97F4A7C15ull

static int g_threads = 1;

void k3g_set_threads(int n) { g_threads = n > 0 ? n : 1; }

uint64_t k3g_mix64(uint64_t z) {
  /* SplitMix64 finaliser (Steele, Lea, Flood 2014; constants of the
   * published generator). */
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t k3g_splitmix64_next(uint64_t *state) {
  *state += K3G_GAMMA;
  return k3g_mix64(*state);
}

uint64_t k3g_draw(uint64_t key, uint64_t i) {
  return k3g_mix64(key + (i + 1u) * K3G_GAMMA);
}

uint64_t k3g_key(uint64_t seed, uint32_t cfg, uint32_t kind, uint32_t a,
                 uint32_t b) {
  uint64_t h = k3g_mix64(seed ^ 0x6B33676B65790001ull);
  h = k3g_mix64(h ^ (((uint64_t)cfg << 32) | kind));
  h = k3g_mix64(h ^ (((uint64_t)a << 32) | b));
  return h;
}

void k3g_bytes(uint64_t key, uint8_t *out, size_t n) {
  const long long nw = (long long)(n / 8);
#pragma omp parallel for num_threads(g_threads) if (n > (1u << 20)) schedule(static)
  for (long long w = 0; w < nw; w++) {
    uint64_t d = k3g_draw(key, (uint64_t)w);
    for (int b = 0; b < 8; b++) out[(size_t)w * 8 + b] = (uint8_t)(d >> (8 * b));
  }
  if (n % 8) {
    uint64_t d = k3g_draw(key, (uint64_t)nw);
    for (size_t b = 0; b < n % 8; b++) out[(size_t)nw * 8 + b] = (uint8_t)(d >> (8 * b));
  }
}

void k3g_uniform_u8(uint64_t key, int lo, int hi, uint8_t *out, size_t n) {
  const uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for num_threads(g_threads) if (n > (1u << 18)) schedule(static)
  for (long long i = 0; i < (long long)n; i++) {
    uint64_t d = k3g_draw(key, (uint64_t)i) >> 32;
    out[i] = (uint8_t)(lo + (int)((d * span) >> 32));
  }
}

static double k3g_std_normal(uint64_t key, size_t i) {
  const size_t j = i / 2;
  const uint64_t d1 = k3g_draw(key, 2 * (uint64_t)j);
  const uint64_t d2 = k3g_draw(key, 2 * (uint64_t)j + 1);
  const double u1 = ((double)(d1 >> 11) + 1.0) * 0x1p-53; /* (0, 1] */
  const double u2 = (double)(d2 >> 11) * 0x1p-53;         /* [0, 1) */
  const double r = sqrt(-2.0 * log(u1));
  const double t = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

void k3g_normal_f32(uint64_t key, double mu, double sigma, float *out,
                    size_t n) {
#pragma omp parallel for num_threads(g_threads) if (n > (1u << 16)) schedule(static)
  for (long long i = 0; i < (long long)n; i++)
    out[i] = (float)(mu + sigma * k3g_std_normal(key, (size_t)i));
}

uint16_t k3g_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void k3g_normal_bf16(uint64_t key, double mu, double sigma, uint16_t *out,
                     size_t n) {
#pragma omp parallel for num_threads(g_threads) if (n > (1u << 16)) schedule(static)
  for (long long i = 0; i < (long long)n; i++) {
    const float f = (float)(mu + sigma * k3g_std_normal(key, (size_t)i));
    out[i] = k3g_f32_to_bf16(f);
  }
}

void k3g_uniform_f32(uint64_t key, float *out, size_t n) {
#pragma omp parallel for num_threads(g_threads) if (n > (1u << 18)) schedule(static)
  for (long long i = 0; i < (long long)n; i++)
    out[i] = (float)(k3g_draw(key, (uint64_t)i) >> 40) * 0x1p-24f;
}

void k3g_mxfp4_matrix(uint64_t seed, uint32_t cfg, uint32_t kind, uint32_t a,
                      uint32_t b, int rows, int cols, int elo, int ehi,
                      uint8_t *nib, uint8_t *sc) {
  const size_t nbytes = (size_t)rows * (size_t)(cols / 2);
  const size_t nsc = (size_t)rows * (size_t)(cols / 32);
  if (nib) k3g_bytes(k3g_key(seed, cfg, kind, a, 2 * b), nib, nbytes);
  if (sc) k3g_uniform_u8(k3g_key(seed, cfg, kind, a, 2 * b + 1), elo, ehi, sc, nsc);
}

void k3g_expert(uint64_t seed, uint32_t cfg, uint32_t expert, int hidden,
                int inter, int elo, int ehi, uint8_t *gate_nib,
                uint8_t *gate_sc, uint8_t *up_nib, uint8_t *up_sc,
                uint8_t *down_nib, uint8_t *down_sc) {
  k3g_mxfp4_matrix(seed, cfg, K3G_KIND_EXPERT, expert, 0, inter, hidden, elo,
                   ehi, gate_nib, gate_sc);
  k3g_mxfp4_matrix(seed, cfg, K3G_KIND_EXPERT, expert, 1, inter, hidden, elo,
                   ehi, up_nib, up_sc);
  k3g_mxfp4_matrix(seed, cfg, K3G_KIND_EXPERT, expert, 2, hidden, inter, elo,
                   ehi, down_nib, down_sc);
}

void k3g_zipf_logits(uint64_t seed, uint32_t cfg, uint32_t batch, int T, int n,
                     double s, float *out) {
  int *perm = (int *)malloc(sizeof(int) * (size_t)n);
  double *lp = (double *)malloc(sizeof(double) * (size_t)n);
  if (!perm || !lp) {
    free(perm);
    free(lp);
    return;
  }
  const uint64_t kp = k3g_key(seed, cfg, K3G_KIND_PERM, 0, 0);
  for (int i = 0; i < n; i++) perm[i] = i;
  for (int i = n - 1; i > 0; i--) { /* Fisher-Yates */
    const uint64_t d = k3g_draw(kp, (uint64_t)(n - 1 - i)) >> 32;
    const int j = (int)((d * (uint64_t)(i + 1)) >> 32);
    const int t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  double z = 0.0;
  for (int r = 1; r <= n; r++) z += pow((double)r, -s);
  /* perm[r-1] is the expert of popularity rank r */
  for (int r = 1; r <= n; r++) lp[perm[r - 1]] = -s * log((double)r) - log(z);
  const uint64_t kg = k3g_key(seed, cfg, K3G_KIND_LOGITS, batch, 0);
#pragma omp parallel for num_threads(g_threads) if ((size_t)T * n > (1u << 16)) schedule(static)
  for (long long i = 0; i < (long long)T * n; i++) {
    const uint64_t d = k3g_draw(kg, (uint64_t)i);
    const double u = ((double)(d >> 11) + 0.5) * 0x1p-53; /* (0, 1) */
    out[i] = (float)(lp[i % n] - log(-log(u)));
  }
  free(perm);
  free(lp);
}
