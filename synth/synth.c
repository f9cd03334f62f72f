/*
 * Seeded synthetic inputs shared by the CPU oracle and the GPU path.
 *
 * This file holds no arithmetic of the QLoRA method: it only turns
 * (seed, stream, index) into pseudo-random numbers.  Both sides of every
 * parity check read the arrays produced here, so they see identical inputs.
 *
 * Generator: the SplitMix64 output function (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), used in
 * counter mode:
 *     key      = mix(seed * GAMMA + stream)
 *     bits(i)  = mix(key + (i + 1) * GAMMA)            (all mod 2^64)
 *     u(i)     = (bits(i) >> 11) * 2^-53               in [0, 1)
 * Normal variates use Box-Muller on two consecutive counters:
 *     z(i)     = sqrt(-2 ln(1 - u(2i))) * cos(2 pi u(2i+1))
 * Every element depends only on its own index, so the loops parallelise
 * trivially and any slice can be regenerated on its own.
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GAMMA + stream);
}

static inline double unit(uint64_t key, uint64_t i) {
  return (double)(mix64(key + (i + 1) * GAMMA) >> 11) * 0x1.0p-53;
}

static inline double normal(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = 1.0 - unit(key, 2 * i);
  double u2 = unit(key, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* fp32 -> bf16, round to nearest even (inputs here are always finite). */
static inline uint16_t f32_to_bf16(float f) {
  union { float f; uint32_t u; } v = {f};
  uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

uint64_t synth_bits(uint64_t seed, uint64_t stream, uint64_t i) {
  return mix64(stream_key(seed, stream) + (i + 1) * GAMMA);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, uint64_t offset,
                      double mean, double std, float* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + std * normal(key, offset + (uint64_t)i));
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, uint64_t offset,
                       double mean, double std, uint16_t* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16((float)(mean + std * normal(key, offset + (uint64_t)i)));
}

void synth_uniform_f32(uint64_t seed, uint64_t stream, int64_t n, uint64_t offset,
                       double lo, double hi, float* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * unit(key, offset + (uint64_t)i));
}

void synth_uniform_bf16(uint64_t seed, uint64_t stream, int64_t n, uint64_t offset,
                        double lo, double hi, uint16_t* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16((float)(lo + (hi - lo) * unit(key, offset + (uint64_t)i)));
}
