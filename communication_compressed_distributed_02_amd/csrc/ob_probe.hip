// Streaming probes of known traffic, for measurement only (they are not part
// of the optimizer step).  bench.py uses them to put the step's kernels next
// to what the memory system delivers for the same access mix on the same
// device, and as plain copy / read / write kernels of known size for scaling
// the profiler's byte counters.
//
// Every probe uses the step's own mapping: a wavefront owns 1024 consecutive
// elements as 16 rows of 64 (lane = column), non-temporal loads and stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 256;

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ int64_t wave_base() {
  return ((int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * 1024;
}

// 6 bytes read + 4 written per element: the worker pass's mix (bf16 in, fp32 in/out).
__global__ void __launch_bounds__(kBlock) mix_kernel(const uint16_t* __restrict__ g,
                                                     float* __restrict__ c) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  float gv[16], cv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    gv[r] = __uint_as_float((uint32_t)ld_nt(g + base + 64 * r + lane) << 16);
    cv[r] = ld_nt(c + base + 64 * r + lane);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) st_nt(c + base + 64 * r + lane, cv[r] * 0.5f + gv[r]);
}

// 8 bytes read + 4 written per element: the worker pass's mix with fp32
// gradients (fp32 in, fp32 in/out).
__global__ void __launch_bounds__(kBlock) mix32_kernel(const float* __restrict__ g,
                                                       float* __restrict__ c) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  float gv[16], cv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    gv[r] = ld_nt(g + base + 64 * r + lane);
    cv[r] = ld_nt(c + base + 64 * r + lane);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) st_nt(c + base + 64 * r + lane, cv[r] * 0.5f + gv[r]);
}

// The 0/1 Adam synchronizing worker pass's mix: gradient (GT), local
// momentum, mean momentum and compensated momentum read, the compensated
// momentum written (gb + 12 B read + 4 B written per element).
template <typename GT>
__device__ __forceinline__ float probe_value(const GT* p, int64_t k);
template <>
__device__ __forceinline__ float probe_value(const uint16_t* p, int64_t k) {
  return __uint_as_float((uint32_t)ld_nt(p + k) << 16);
}
template <>
__device__ __forceinline__ float probe_value(const float* p, int64_t k) {
  return ld_nt(p + k);
}
template <typename GT>
__global__ void __launch_bounds__(kBlock) sync_mix_kernel(const GT* __restrict__ g,
                                                          const float* __restrict__ m,
                                                          const float* __restrict__ a,
                                                          float* __restrict__ c) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t k = base + 64 * r + lane;
    st_nt(c + k, ((probe_value(g, k) + ld_nt(m + k)) + ld_nt(a + k)) * 0.5f + ld_nt(c + k));
  }
}

// 4 bytes read + 4 written per element: a plain copy.
__global__ void __launch_bounds__(kBlock) copy_kernel(const float* __restrict__ a,
                                                      float* __restrict__ b) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = ld_nt(a + base + 64 * r + lane);
#pragma unroll
  for (int r = 0; r < 16; ++r) st_nt(b + base + 64 * r + lane, v[r]);
}

// 4 bytes read per element (one float per wave written when the data hits a
// value that never occurs, which keeps the loads live).
__global__ void __launch_bounds__(kBlock) read_kernel(const float* __restrict__ a,
                                                      float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
  float acc = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc += ld_nt(a + base + 64 * r + lane);
  if (acc == -1.0e30f) sink[0] = acc;
}

// 4 bytes written per element.
__global__ void __launch_bounds__(kBlock) write_kernel(float* __restrict__ b) {
  const int lane = threadIdx.x & 63;
  const int64_t base = wave_base();
#pragma unroll
  for (int r = 0; r < 16; ++r) st_nt(b + base + 64 * r + lane, (float)r);
}

}  // namespace

// kind: 0 = mix (a: bf16 elements, b: fp32 elements), 1 = copy a -> b (fp32),
// 2 = read a (fp32; b receives at most one float), 3 = write b (fp32),
// 4 = mix with fp32 a.
// n: elements, a positive multiple of 4096 (whole blocks); returns 0 on
// success, 1 for bad arguments, 2 for a launch error.
extern "C" int ob_probe_run(int kind, const void* a, void* b, int64_t n, void* stream) {
  if (n <= 0 || n % 4096 != 0 || kind < 0 || kind > 4) return 1;
  if ((kind != 3 && a == nullptr) || b == nullptr) return 1;
  const int64_t blocks = n / 4096;
  if (blocks > 0x7fffffff) return 1;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)blocks), block(kBlock);
  switch (kind) {
    case 0: mix_kernel<<<grid, block, 0, s>>>((const uint16_t*)a, (float*)b); break;
    case 1: copy_kernel<<<grid, block, 0, s>>>((const float*)a, (float*)b); break;
    case 2: read_kernel<<<grid, block, 0, s>>>((const float*)a, (float*)b); break;
    case 3: write_kernel<<<grid, block, 0, s>>>((float*)b); break;
    case 4: mix32_kernel<<<grid, block, 0, s>>>((const float*)a, (float*)b); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The synchronizing-pass mix over n elements (a positive multiple of 4096):
// g holds bf16 (bf16 != 0) or fp32 gradients; m, a, c fp32.  Same returns as
// ob_probe_run.
extern "C" int ob_probe_run_sync(int bf16, const void* g, const float* m, const float* a,
                                 float* c, int64_t n, void* stream) {
  if (n <= 0 || n % 4096 != 0 || g == nullptr || m == nullptr || a == nullptr || c == nullptr)
    return 1;
  const int64_t blocks = n / 4096;
  if (blocks > 0x7fffffff) return 1;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)blocks), block(kBlock);
  if (bf16)
    sync_mix_kernel<uint16_t><<<grid, block, 0, s>>>((const uint16_t*)g, m, a, c);
  else
    sync_mix_kernel<float><<<grid, block, 0, s>>>((const float*)g, m, a, c);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
