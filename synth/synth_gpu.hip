// Device side of the seeded gradient generator.  See philox.h for the
// definition; synth_cpu.c produces the same bits on the host.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#define SYNTH_QUAL __device__ static inline
#include "philox.h"

template <int DTYPE>
__global__ void __launch_bounds__(256) synth_fill_kernel(void* __restrict__ out, int64_t count,
                                                         uint64_t elem0, uint32_t step,
                                                         uint32_t seed, uint32_t worker, int dist,
                                                         float k, float sigma) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    float v = synth_value(dist, elem0 + (uint64_t)i, step, seed, worker, k, sigma);
    if (DTYPE == 0)
      ((float*)out)[i] = v;
    else
      ((uint16_t*)out)[i] = synth_to_bf16(v);
  }
}

extern "C" int synth_fill_device(void* out, int dtype, int64_t count, uint64_t elem0,
                                 uint32_t step, uint32_t seed, uint32_t worker, int dist, float k,
                                 float sigma, void* stream) {
  if (count <= 0) return 0;
  if (out == nullptr || (dtype != 0 && dtype != 1) || (dist != 0 && dist != 1)) return 1;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == 0)
    synth_fill_kernel<0><<<(unsigned)blocks, 256, 0, s>>>(out, count, elem0, step, seed, worker,
                                                          dist, k, sigma);
  else
    synth_fill_kernel<1><<<(unsigned)blocks, 256, 0, s>>>(out, count, elem0, step, seed, worker,
                                                          dist, k, sigma);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
