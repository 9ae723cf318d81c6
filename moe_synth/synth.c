/*
 * Seeded synthetic inputs for the MoE expert-layer path.
 *
 * This file holds no arithmetic of the MoE method itself: it only draws the
 * tensors the method consumes (token activations, router and expert weights,
 * per-expert logit bias, upstream gradients).  Both the CPU oracle and the GPU
 * path read what it writes, so the two always see bit-identical inputs.
 *
 * Generator (a definition, so that any element can be re-derived alone):
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014) used in counter mode: draw n of stream key K is
 *     mix64(K + (n + 1) * 0x9E3779B97F4A7C15), mix64 being its output
 *     finaliser.
 *   - stream key K = mix64(mix64(seed) ^ (stream * 0xD1B54A32D192ED03)).
 *   - normal deviates by the Box-Muller transform (Box & Muller 1958) in fp64:
 *     element i uses draws 2*(i/2) and 2*(i/2)+1 as u1 in (0,1], u2 in [0,1);
 *     even i take r*cos(2*pi*u2), odd i take r*sin(2*pi*u2), r = sqrt(-2 ln u1).
 *   - value = mean + std * z in fp64, rounded to fp32 (round-to-nearest-even),
 *     and for bf16 outputs further rounded fp32 -> bf16 (round-to-nearest-even).
 * Element indices are global within a tensor, so a slice (for example the
 * first n experts of a stacked weight tensor) has the same values as the
 * corresponding part of the whole tensor.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t n) {
  return mix64(key + (n + 1) * kGolden);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  uint64_t h1 = draw(key, 2 * p), h2 = draw(key, 2 * p + 1);
  double u1 = (double)((h1 >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)(h2 >> 11) * 0x1.0p-53;       /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline void normal_pair(uint64_t key, uint64_t p, double *z0,
                               double *z1) {
  uint64_t h1 = draw(key, 2 * p), h2 = draw(key, 2 * p + 1);
  double u1 = (double)((h1 >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(h2 >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(th);
  *z1 = r * sin(th);
}

/* Elements [offset, offset + n) of a stream, both Box-Muller outputs of each
 * pair used; identical values to normal_at(). */
#define SYNTH_FILL(CONVERT)                                                  \
  uint64_t key = synth_stream_key(seed, stream);                             \
  uint64_t p0 = offset >> 1, p1 = (offset + n + 1) >> 1;                     \
  _Pragma("omp parallel for schedule(static, 32768)")                        \
  for (int64_t p = (int64_t)p0; p < (int64_t)p1; ++p) {                      \
    double z[2];                                                             \
    normal_pair(key, (uint64_t)p, &z[0], &z[1]);                             \
    for (int q = 0; q < 2; ++q) {                                            \
      uint64_t i = 2 * (uint64_t)p + (uint64_t)q;                            \
      if (i < offset || i >= offset + n) continue;                           \
      out[i - offset] = CONVERT((float)(mean + std * z[q]));                 \
    }                                                                        \
  }

#define SYNTH_ID(v) (v)

/* out[j] = fp32(mean + std * z(offset + j)), j < n */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset,
                      uint64_t n, double mean, double std, float *out) {
  SYNTH_FILL(SYNTH_ID)
}

/* out[j] = bf16(fp32(mean + std * z(offset + j))) as raw bits, j < n */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset,
                       uint64_t n, double mean, double std, uint16_t *out) {
  SYNTH_FILL(f32_to_bf16_rne)
}

/* A seeded permutation of 0..n-1 (Fisher-Yates, draw j picks among i+1). */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t *out) {
  uint64_t key = synth_stream_key(seed, stream);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t h = draw(key, (uint64_t)i);
    int32_t j = (int32_t)(((__uint128_t)h * (uint64_t)(i + 1)) >> 64);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* Per-expert Zipf logit bias.  A seeded shuffle lists the experts from
 * most to least popular: the expert at position i has rank i + 1 and bias
 * b = (i + 1)^(-s), in fp64. */
void synth_zipf_bias(uint64_t seed, uint64_t stream, int32_t n_experts,
                     double s, double *out) {
  int32_t order[4096];
  if (n_experts > 4096) return;
  synth_permutation(seed, stream, n_experts, order);
  for (int32_t i = 0; i < n_experts; ++i)
    out[order[i]] = pow(1.0 + (double)i, -s);
}

/* Gaussian logits plus a per-expert bias: out[t*E+e] = fp32(z + bias[e]). */
void synth_biased_logits(uint64_t seed, uint64_t stream, int64_t T, int32_t E,
                         const double *bias, float *out) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static, 64)
  for (int64_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e) {
      uint64_t i = (uint64_t)t * (uint64_t)E + (uint64_t)e;
      out[i] = (float)(normal_at(key, i) + (bias ? bias[e] : 0.0));
    }
}
