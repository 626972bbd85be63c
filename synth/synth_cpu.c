/* Host side of the seeded gradient generator (plain C).  See philox.h for the
 * definition; the GPU side (synth_gpu.hip) produces the same bits. */
#include <math.h>
#include <stdint.h>

#define SYNTH_QUAL static inline
#include "philox.h"

void synth_philox_block(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                        uint32_t k1, uint32_t* out4) {
  synth_u32x4 r = synth_philox4x32_10(c0, c1, c2, c3, k0, k1);
  for (int i = 0; i < 4; ++i) out4[i] = r.v[i];
}

/* out[i] = value of element (elem0 + i); dtype 0 = fp32, 1 = bf16 bits. */
void synth_fill(void* out, int dtype, int64_t count, uint64_t elem0, uint32_t step, uint32_t seed,
                uint32_t worker, int dist, float k, float sigma) {
  if (dtype == 0) {
    float* o = (float*)out;
    for (int64_t i = 0; i < count; ++i)
      o[i] = synth_value(dist, elem0 + (uint64_t)i, step, seed, worker, k, sigma);
  } else {
    uint16_t* o = (uint16_t*)out;
    for (int64_t i = 0; i < count; ++i)
      o[i] = synth_to_bf16(synth_value(dist, elem0 + (uint64_t)i, step, seed, worker, k, sigma));
  }
}

/* Same values at an explicit list of element indices (sampled checks). */
void synth_gather(void* out, int dtype, int64_t count, const uint64_t* elems, uint32_t step,
                  uint32_t seed, uint32_t worker, int dist, float k, float sigma) {
  if (dtype == 0) {
    float* o = (float*)out;
    for (int64_t i = 0; i < count; ++i)
      o[i] = synth_value(dist, elems[i], step, seed, worker, k, sigma);
  } else {
    uint16_t* o = (uint16_t*)out;
    for (int64_t i = 0; i < count; ++i)
      o[i] = synth_to_bf16(synth_value(dist, elems[i], step, seed, worker, k, sigma));
  }
}
