// Elementwise checks of the floating-point environment the step's kernels
// are compiled with (the same flags as libob_adam.so): correctly rounded
// fp32 square root and division, fp64 square root and division, fp64 -> fp32
// conversion, no flush of denormals, and no contraction of a multiply and an
// add into one fused operation.  Used by the tests, which compare every
// result bit for bit with the host's IEEE arithmetic; not part of the step.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 256;

template <typename F>
__global__ void __launch_bounds__(kBlock) map_kernel(int64_t n, F f) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) f(i);
}

}  // namespace

// op 0: out = sqrtf(a)            (a, out fp32)
// op 1: out = a / b               (fp32)
// op 2: out = sqrt(a)             (fp64)
// op 3: out = a / b               (fp64)
// op 4: out = (float)a            (a fp64, out fp32)
// op 5: out = (a * b) + a         (fp32; must round twice)
// n elements in each array, a positive count.  Returns 0 on success, 1 for
// bad arguments, 2 for a launch error.
extern "C" int ob_mathcheck_run(int op, const void* a, const void* b, void* out, int64_t n,
                                void* stream) {
  if (n <= 0 || op < 0 || op > 5 || a == nullptr || out == nullptr) return 1;
  if ((op == 1 || op == 3 || op == 5) && b == nullptr) return 1;
  hipStream_t s = (hipStream_t)stream;
  int64_t blocks = (n + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks), block(kBlock);
  const float* af = (const float*)a;
  const float* bf = (const float*)b;
  const double* ad = (const double*)a;
  const double* bd = (const double*)b;
  float* of = (float*)out;
  double* od = (double*)out;
  switch (op) {
    case 0: map_kernel<<<grid, block, 0, s>>>(n, [=] __device__(int64_t i) { of[i] = sqrtf(af[i]); }); break;
    case 1: map_kernel<<<grid, block, 0, s>>>(n, [=] __device__(int64_t i) { of[i] = af[i] / bf[i]; }); break;
    case 2: map_kernel<<<grid, block, 0, s>>>(n, [=] __device__(int64_t i) { od[i] = sqrt(ad[i]); }); break;
    case 3: map_kernel<<<grid, block, 0, s>>>(n, [=] __device__(int64_t i) { od[i] = ad[i] / bd[i]; }); break;
    case 4: map_kernel<<<grid, block, 0, s>>>(n, [=] __device__(int64_t i) { of[i] = (float)ad[i]; }); break;
    case 5: map_kernel<<<grid, block, 0, s>>>(n, [=] __device__(int64_t i) { of[i] = (af[i] * bf[i]) + af[i]; }); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
