/*
 * Seeded synthetic-gradient generator (input generation only; it holds none
 * of the optimizer's arithmetic).
 *
 * Counter-based so that any element of any worker's gradient at any step can
 * be produced on its own, on the host (synth_cpu.c, plain C) and on the GPU
 * (synth_gpu.hip), bit-identically.  The includer defines SYNTH_QUAL first
 * (e.g. "static inline" on the host, "__device__ static inline" in HIP).
 *
 * Philox4x32-10 follows its published definition: Salmon, Moraes, Dror,
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11, section 4.2
 * (multipliers 0xD2511F53 / 0xCD9E8D57, Weyl key increments 0x9E3779B9 /
 * 0xBB67AE85, ten rounds).
 *
 * Counter layout: (element index lo, element index hi, step, draw); key:
 * (seed, worker).  "draw" separates the independent normals a Student-t
 * sample needs.
 *
 * Normal: Irwin-Hall sum of four 24-bit uniforms taken from one Philox block,
 * centred as an integer (2*sum - (2^26 - 4)), converted once to fp32 (round to
 * nearest even on both sides) and multiplied by a caller-provided fp32 scale.
 * With scale = sigma*sqrt(3)/2^25 the result has standard deviation sigma.
 * No transcendental function is involved, so host and device agree exactly.
 *
 * Student-t, 3 degrees of freedom: z0 / sqrtf(((z1*z1 + z2*z2) + z3*z3) / 3)
 * from four unit normals (draws 0..3), times sigma; 0 when the denominator is 0.
 * sqrtf and '/' must be correctly rounded on both sides.
 *
 * bf16: fp32 rounded to nearest even on the bit pattern (no NaN can occur).
 */
#ifndef SYNTH_PHILOX_H
#define SYNTH_PHILOX_H

#include <stdint.h>

#ifndef SYNTH_QUAL
#error "define SYNTH_QUAL before including philox.h"
#endif

#define SYNTH_PHILOX_M0 0xD2511F53u
#define SYNTH_PHILOX_M1 0xCD9E8D57u
#define SYNTH_PHILOX_W0 0x9E3779B9u
#define SYNTH_PHILOX_W1 0xBB67AE85u

/* distributions */
#define SYNTH_NORMAL 0
#define SYNTH_STUDENT_T3 1

typedef struct { uint32_t v[4]; } synth_u32x4;

SYNTH_QUAL synth_u32x4 synth_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                          uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += SYNTH_PHILOX_W0; k1 += SYNTH_PHILOX_W1; }
    uint64_t p0 = (uint64_t)SYNTH_PHILOX_M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)SYNTH_PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  synth_u32x4 out;
  out.v[0] = c0; out.v[1] = c1; out.v[2] = c2; out.v[3] = c3;
  return out;
}

/* Centred Irwin-Hall(4) integer in [-(2^26-4), 2^26-4]. */
SYNTH_QUAL int32_t synth_ih4(uint64_t elem, uint32_t step, uint32_t draw, uint32_t seed,
                             uint32_t worker) {
  synth_u32x4 r = synth_philox4x32_10((uint32_t)elem, (uint32_t)(elem >> 32), step, draw, seed,
                                      worker);
  int32_t sum = (int32_t)(r.v[0] >> 8) + (int32_t)(r.v[1] >> 8) + (int32_t)(r.v[2] >> 8) +
                (int32_t)(r.v[3] >> 8);
  return 2 * sum - ((1 << 26) - 4);
}

/* One gradient value in fp32.  k = fp32 scale of the integer normal
 * (sigma*sqrt(3)/2^25 for a normal; sqrt(3)/2^25 for the Student-t's normals),
 * sigma = fp32 multiplier applied to the Student-t ratio (unused for normal). */
SYNTH_QUAL float synth_value(int dist, uint64_t elem, uint32_t step, uint32_t seed, uint32_t worker,
                             float k, float sigma) {
  if (dist == SYNTH_NORMAL) {
    return (float)synth_ih4(elem, step, 0u, seed, worker) * k;
  }
  float z0 = (float)synth_ih4(elem, step, 0u, seed, worker) * k;
  float z1 = (float)synth_ih4(elem, step, 1u, seed, worker) * k;
  float z2 = (float)synth_ih4(elem, step, 2u, seed, worker) * k;
  float z3 = (float)synth_ih4(elem, step, 3u, seed, worker) * k;
  float q = ((z1 * z1) + (z2 * z2)) + (z3 * z3);
  float den = sqrtf(q / 3.0f);
  if (den == 0.0f) return 0.0f;
  return (z0 / den) * sigma;
}

SYNTH_QUAL uint16_t synth_to_bf16(float f) {
  union { float f; uint32_t u; } cv;
  cv.f = f;
  uint32_t lsb = (cv.u >> 16) & 1u;
  uint32_t r = cv.u + 0x7FFFu + lsb;
  return (uint16_t)(r >> 16);
}

#endif
