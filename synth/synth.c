/*
 * synth.c -- seeded synthetic inputs for the fused MoE forward.
 *
 * This module holds none of the method's arithmetic: it only draws numbers.
 * Both the CPU oracle's tests and the GPU benchmark take their inputs from
 * here, so the two sides see the same bytes.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; the finaliser constants of
 * Vigna's public-domain splitmix64.c), used counter-style: draw i of a
 * stream is mix(key + (i + 1) * golden_gamma), so any range of a tensor can
 * be generated in parallel and the result does not depend on thread count.
 * Normals: Box-Muller (1958) on pairs of uniforms.
 *
 * Router (an input of the forward pass, not part of it): softmax over all
 * experts' logits in fp64, top-k by value (ties to the lower expert id),
 * weights renormalised over the k chosen, stored as fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static const uint64_t GOLDEN_GAMMA = 0x9E3779B97F4A7C15ULL;

uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(seed * GOLDEN_GAMMA + synth_mix64(stream + 0x5EEDULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return synth_mix64(key + (i + 1) * GOLDEN_GAMMA);
}

/* uniform in (0, 1): 53 random bits, offset by half a unit */
static inline double unif(uint64_t key, uint64_t i) {
  return ((double)(draw(key, i) >> 11) + 0.5) * 0x1p-53;
}

static inline void normal_pair(uint64_t key, int64_t pair, double* n0, double* n1) {
  double u1 = unif(key, (uint64_t)(2 * pair));
  double u2 = unif(key, (uint64_t)(2 * pair + 1));
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586 * u2;
  *n0 = r * cos(th);
  *n1 = r * sin(th);
}

/* round-to-nearest-even of an fp32 value to bf16 bits */
static inline uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* n normals of mean `mean` and standard deviation `std`, as fp32 */
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double mean, double std, float* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; p++) {
    double a, b;
    normal_pair(key, p, &a, &b);
    out[2 * p] = (float)(mean + std * a);
    if (2 * p + 1 < n) out[2 * p + 1] = (float)(mean + std * b);
  }
}

/* the same draws, stored as bf16 (the fp32 value rounded to nearest even) */
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double mean, double std, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; p++) {
    double a, b;
    normal_pair(key, p, &a, &b);
    out[2 * p] = to_bf16((float)(mean + std * a));
    if (2 * p + 1 < n) out[2 * p + 1] = to_bf16((float)(mean + std * b));
  }
}

/* raw 64-bit draws (tests of the generator itself) */
void synth_u64(uint64_t seed, uint64_t stream, int64_t n, uint64_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; i++) out[i] = draw(key, (uint64_t)i);
}

/* Router: z = logits (+ bias[e] when bias != NULL).  Choose the k largest z
 * (ties to the lower id), weights exp(z_j - zmax) / sum over the chosen. */
void synth_router(const float* logits, const float* bias, int64_t M, int E, int k, int32_t* ids, float* weights) {
#pragma omp parallel
  {
    double* z = (double*)malloc((size_t)E * sizeof(double));
    unsigned char* used = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < M; t++) {
      double zmax = -INFINITY;
      for (int e = 0; e < E; e++) {
        z[e] = (double)logits[t * E + e] + (bias ? (double)bias[e] : 0.0);
        if (z[e] > zmax) zmax = z[e];
        used[e] = 0;
      }
      double sum = 0.0;
      double sel[64];
      for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++)
          if (!used[e] && (best < 0 || z[e] > z[best])) best = e;
        used[best] = 1;
        ids[t * k + j] = best;
        sel[j] = exp(z[best] - zmax);
        sum += sel[j];
      }
      for (int j = 0; j < k; j++) weights[t * k + j] = (float)(sel[j] / sum);
    }
    free(z);
    free(used);
  }
}

/* n distinct token indices in [0, M): always 0 and M-1, the rest drawn by a
 * partial Fisher-Yates shuffle; returned in ascending order. */
void synth_sample_tokens(uint64_t seed, int64_t M, int n, int32_t* out) {
  if (n > M) n = (int)M;
  int32_t* perm = (int32_t*)malloc((size_t)M * sizeof(int32_t));
  for (int64_t i = 0; i < M; i++) perm[i] = (int32_t)i;
  uint64_t key = stream_key(seed, 99);
  int taken = 0;
  /* put 0 and M-1 first */
  if (n > 0) { taken = 1; }
  if (n > 1 && M > 1) { int32_t tmp = perm[1]; perm[1] = perm[M - 1]; perm[M - 1] = tmp; taken = 2; }
  for (int i = taken; i < n; i++) {
    int64_t span = M - i;
    int64_t j = i + (int64_t)(draw(key, (uint64_t)i) % (uint64_t)span);
    int32_t tmp = perm[i]; perm[i] = perm[j]; perm[j] = tmp;
  }
  for (int i = 0; i < n; i++) out[i] = perm[i];
  /* ascending order */
  for (int i = 1; i < n; i++) {
    int32_t v = out[i];
    int j = i - 1;
    while (j >= 0 && out[j] > v) { out[j + 1] = out[j]; j--; }
    out[j + 1] = v;
  }
  free(perm);
}
