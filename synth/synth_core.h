/*
 * Counter-based seeded generator for synthetic inputs (weights, activations,
 * token ids, KV-cache contents).
 *
 * This module holds no part of the decoder arithmetic.  It is shared by the
 * CPU oracle side and the GPU side so that both see bit-identical inputs:
 * the host build (g++) and the device build (hipcc) compile this same header.
 *
 * Definition (every step is integer arithmetic or a correctly rounded IEEE
 * operation, so host and device produce identical bits):
 *   mix(z)        SplitMix64 finaliser (Steele, Lea, Flood 2014).
 *   key           mix(seed * 0x100000001B3 ^ stream)
 *   stream        FNV-1a 64 of the tensor name (computed on the host).
 *   normal(i)     three 64-bit words w_j = mix(key + 3*i + j), j = 0..2, give
 *                 twelve 16-bit uniforms u_0..u_11 in [0, 65535];
 *                 S = sum u_k; z = (2*S - 786420) / 2^17.
 *                 This is the Irwin-Hall(12) approximation of N(0,1): mean 0,
 *                 variance 1 - 2^-32, support [-6, 6].  2*S - 786420 is an
 *                 integer below 2^20, so z is exact in fp32.
 *   value         bf16_rne(float(double(mean) + double(std) * double(z))).
 *                 std*z is exact in double (24 + 20 significant bits), so a
 *                 fused multiply-add and a separate multiply and add agree.
 *   uniform(i)    lo + ((mix(key + i) >> 32) * (hi - lo)) >> 32.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifdef __HIPCC__
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

SYNTH_FN uint64_t synth_mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix(seed * 0x100000001B3ull ^ stream);
}

SYNTH_FN uint32_t synth_sum16(uint64_t w) {
  return (uint32_t)(w & 0xFFFF) + (uint32_t)((w >> 16) & 0xFFFF) +
         (uint32_t)((w >> 32) & 0xFFFF) + (uint32_t)(w >> 48);
}

/* Standard-normal approximation for counter i (exact fp32 value). */
SYNTH_FN float synth_z(uint64_t key, uint64_t i) {
  uint64_t base = key + 3ull * i;
  uint32_t s = synth_sum16(synth_mix(base)) + synth_sum16(synth_mix(base + 1)) +
               synth_sum16(synth_mix(base + 2));
  int32_t t = 2 * (int32_t)s - 786420;
  return (float)t * (1.0f / 131072.0f);
}

SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

SYNTH_FN uint16_t synth_normal_bf16_at(uint64_t key, uint64_t i, float mean, float stdv) {
  double y = (double)mean + (double)stdv * (double)synth_z(key, i);
  return synth_f32_to_bf16((float)y);
}

SYNTH_FN int32_t synth_uniform_at(uint64_t key, uint64_t i, int32_t lo, int32_t hi) {
  uint64_t w = synth_mix(key + i) >> 32;
  uint64_t range = (uint64_t)((int64_t)hi - (int64_t)lo);
  return (int32_t)((int64_t)lo + (int64_t)((w * range) >> 32));
}

#endif
