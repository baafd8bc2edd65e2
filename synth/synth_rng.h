/*
 * synth_rng.h - seeded, counter-based input generator shared by the CPU and GPU
 * builds of the synthetic-input module.
 *
 * This header holds no part of the loss method: it only turns (seed, stream,
 * index) into bits and the bits into synthetic values.  It is compiled twice,
 * by gcc for the host library and by hipcc for the device library, and every
 * value it produces is bit-identical on both because it uses integer
 * arithmetic plus one IEEE binary64 multiply and one round-to-nearest-even
 * narrowing per element (no transcendental functions, no contraction).
 *
 * Bits: the SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; finaliser constants of
 * Stafford's "Mix13") applied to key + (counter + 1) * golden-gamma.
 *
 * Normal values: the Irwin-Hall(12) approximation of N(0,1), i.e. the sum of
 * twelve uniforms minus six.  Each uniform is a 16-bit field b of a draw,
 * taken as (b + 1/2) / 65536, so the sum minus six is the exact dyadic number
 * (sum(b) - 393210) / 65536: mean 0, variance 1 - 2^-32, support +-6.
 */
#ifndef SYNTH_RNG_H
#define SYNTH_RNG_H

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL
#define SYNTH_STREAM_SALT 0x632BE59BD9B4E019ULL

/* SplitMix64 output (mixing) function. */
SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of one (seed, stream) pair: independent streams of the same seed. */
SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix64(synth_mix64(seed) ^ (stream * SYNTH_GAMMA + SYNTH_STREAM_SALT));
}

/* Draw number `counter` of a stream. */
SYNTH_FN uint64_t synth_draw(uint64_t key, uint64_t counter) {
  return synth_mix64(key + (counter + 1ULL) * SYNTH_GAMMA);
}

/* Irwin-Hall(12) numerator of element `idx`: the normal value is num / 65536. */
SYNTH_FN int32_t synth_ih12_num(uint64_t key, uint64_t idx) {
  int32_t s = 0;
  for (int k = 0; k < 3; ++k) {
    uint64_t d = synth_draw(key, 3ULL * idx + (uint64_t)k);
    s += (int32_t)(d & 0xFFFFu) + (int32_t)((d >> 16) & 0xFFFFu) +
         (int32_t)((d >> 32) & 0xFFFFu) + (int32_t)(d >> 48);
  }
  return s - 393210;
}

/* Element `idx` of N(0, std^2) (Irwin-Hall approximation) as a binary32: the
 * numerator scaled by 2^-16 is exact, the multiply by std is one binary64
 * rounding and the narrowing to binary32 is one more. */
SYNTH_FN float synth_normal_f32(uint64_t key, uint64_t idx, double stdev) {
  double z = (double)synth_ih12_num(key, idx) * (1.0 / 65536.0);
  double v = z * stdev; /* one rounded multiply; nothing to contract with */
  return (float)v;
}

/* binary32 -> bfloat16 bits, round to nearest even (finite inputs). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif /* SYNTH_RNG_H */
