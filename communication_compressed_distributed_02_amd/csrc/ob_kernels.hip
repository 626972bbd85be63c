// gfx950 kernels of the 1-bit Adam compressed step.
//
// Method: "1-bit Adam: Communication Efficient Large-Scale Training with
// Adam's Convergence Speed" (Abstract) and "LIT-278: 1-bit Adam ..." (Key
// takeaways: 1-bit compressed momentum SGD preconditioned by the frozen
// variance; Theorem 1 conditions: error-compensated 1-bit compression with
// per-chunk scaling; tag lines SOTA-214 and SOTA-215).  The arithmetic
// contract these kernels implement is stated in include/ob_adam.h.
//
// Layout and mapping (wave64 throughout):
//  - A "segment" is 1024 consecutive elements of one chunk, seen as 16 rows
//    of 64; one wavefront owns a segment and lane k owns column k.  Every
//    load and store of a row is one fully coalesced 256-byte (fp32) or
//    128-byte (bf16) access, the row's sign word is one ballot, and lane k's
//    fp64 accumulator over the 16 rows followed by an xor butterfly is
//    exactly the fixed summation order of the contract.
//  - Errors are not stored: a worker keeps its last compensated momentum c
//    and a server its last u, and the error c - (c >= 0 ? s : -s) is formed
//    in registers when the next step reads c.  The subtraction is the same
//    fp32 operation the eager form would do, so the values are identical,
//    and each step reads and writes one fp32 array per worker instead of
//    two passes.
//  - After the first compressed step the momentum is exactly the
//    decompressed server output, so it is kept as the server's sign words and
//    per-chunk scales (1/8 byte per element instead of 4 read + 4 written).
//  - Sign words are read with scalar (uniform) loads and decoded with an
//    inverse ballot: bit `lane` of a uniform 64-bit word selects +s or -s in
//    one v_cndmask.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ob_kernels.h"

namespace ob {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;

// Index of this wavefront in its block, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ float grad_value(const float* g, int64_t k) { return g[k]; }
__device__ __forceinline__ float grad_value(const uint16_t* g, int64_t k) {
  return __uint_as_float((uint32_t)g[k] << 16);  // bf16 -> fp32, exact
}

// +s where bit `lane` of the uniform word is set, -s elsewhere.
__device__ __forceinline__ float signed_scale(uint64_t word, float s) {
  return __builtin_amdgcn_inverse_ballot_w64(word) ? s : -s;
}

// acc + c*c with the square exact in fp64, so the fused form rounds once
// exactly like the separate add of the exact square.
__device__ __forceinline__ double add_square(double acc, float c) {
  double cd = (double)c;
  return __builtin_fma(cd, cd, acc);
}

// xor butterfly over the 64 lanes, offsets 32, 16, 8, 4, 2, 1.
__device__ __forceinline__ double butterfly(double acc) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o, 64);
  return acc;
}

// Pairwise sum by levels of N values (N a power of two), in place.
template <int N>
__device__ __forceinline__ float pairwise_sum(float* v) {
#pragma unroll
  for (int h = N / 2; h >= 1; h /= 2) {
#pragma unroll
    for (int i = 0; i < h; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  }
  return v[0];
}

// Pairwise sum by levels for any n <= 64 (an odd tail passes up).
__device__ __forceinline__ float pairwise_sum_any(float* v, int n) {
  int cnt = n;
  while (cnt > 1) {
    int half = cnt >> 1;
    for (int i = 0; i < half; ++i) v[i] = v[2 * i] + v[2 * i + 1];
    if (cnt & 1) {
      v[half] = v[cnt - 1];
      cnt = half + 1;
    } else {
      cnt = half;
    }
  }
  return v[0];
}

// ----------------------------------------------------------------- warm-up --
// Full-precision Adam with bias correction on the pairwise worker average.
template <typename GT, int NW>
__global__ void __launch_bounds__(kBlock)
    warmup_kernel(GradPtrs g, int n, int64_t d, float* __restrict__ m, float* __restrict__ v,
                  float* __restrict__ x, float beta1, float ob1, float beta2, float ob2, float bc1,
                  float bc2, float lr, float eps) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < d; k += stride) {
    float vals[NW > 0 ? NW : kMaxWorkersPerLaunch];
    float sum;
    if constexpr (NW > 0) {
#pragma unroll
      for (int w = 0; w < NW; ++w) vals[w] = grad_value((const GT*)g.p[w], k);
      sum = pairwise_sum<NW>(vals);
    } else {
      for (int w = 0; w < n; ++w) vals[w] = grad_value((const GT*)g.p[w], k);
      sum = pairwise_sum_any(vals, n);
    }
    const float gbar = sum / (float)(NW > 0 ? NW : n);
    const float mk = (beta1 * m[k]) + (ob1 * gbar);
    const float vk = (beta2 * v[k]) + (ob2 * (gbar * gbar));
    m[k] = mk;
    v[k] = vk;
    const float mh = mk / bc1;
    const float vh = vk / bc2;
    x[k] = x[k] - lr * (mh / (sqrtf(vh) + eps));
  }
}

// ------------------------------------------------------------- worker pass --
// c = ((b1*m) + ((1-b1)*g)) + e with e = c_prev - (c_prev >= 0 ? s_prev : -s_prev);
// stores c, the row's sign word and the segment's fp64 sum of squares.
// grid.y = (worker in launch) * n + chunk; grid.x strides over segments.
template <typename GT, bool MBITS>
__device__ __forceinline__ void worker_row(const GT* __restrict__ g, float* __restrict__ c,
                                           const float* __restrict__ m, uint64_t mword, float ms,
                                           int64_t k, float sp, float beta1, float ob1,
                                           double& acc, uint64_t& word) {
  const float gv = grad_value(g, k);
  const float cp = c[k];
  const float e = cp - (cp >= 0.0f ? sp : -sp);
  const float mv = MBITS ? signed_scale(mword, ms) : m[k];
  const float cv = ((beta1 * mv) + (ob1 * gv)) + e;
  c[k] = cv;
  word = __ballot(cv >= 0.0f);
  acc = add_square(acc, cv);
}

template <typename GT, bool MBITS>
__global__ void __launch_bounds__(kBlock)
    worker_kernel(GradPtrs g, int w0, int64_t d, int64_t L, int n, int64_t nseg, int64_t words,
                  const float* __restrict__ m, const uint64_t* __restrict__ sbits,
                  const float* __restrict__ sscale, float* __restrict__ cbuf,
                  const float* __restrict__ wscale, uint64_t* __restrict__ wbits,
                  double* __restrict__ wpart, float beta1, float ob1) {
  const int lane = threadIdx.x & 63;
  const int wi = (int)blockIdx.y / n;  // worker within this launch
  const int j = (int)blockIdx.y - wi * n;
  const int w = w0 + wi;
  const GT* __restrict__ gp = (const GT*)g.p[wi];
  float* __restrict__ c = cbuf + (int64_t)w * d;
  uint64_t* __restrict__ bits = wbits + (int64_t)w * words;
  const float sp = wscale[w * n + j];  // this worker's scale of chunk j, previous step
  const float ms = MBITS ? sscale[j] : 0.0f;
  const int64_t nwave = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t s = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block(); s < nseg;
       s += nwave) {
    const int64_t q0 = s * kSegElems;
    const int64_t left = (L - q0) >> 6;
    const int rows = left < kSegRows ? (int)left : kSegRows;
    const int64_t base = (int64_t)j * L + q0;  // global index of the segment's first element
    const int64_t wbase = base >> 6;
    double acc = 0.0;
    uint64_t mine = 0;
    if (rows == kSegRows) {
#pragma unroll
      for (int r = 0; r < kSegRows; ++r) {
        uint64_t word;
        const uint64_t mword = MBITS ? sbits[wbase + r] : 0;
        worker_row<GT, MBITS>(gp, c, m, mword, ms, base + 64 * r + lane, sp, beta1, ob1, acc,
                              word);
        mine = lane == r ? word : mine;
      }
    } else {
      for (int r = 0; r < rows; ++r) {
        uint64_t word;
        const uint64_t mword = MBITS ? sbits[wbase + r] : 0;
        worker_row<GT, MBITS>(gp, c, m, mword, ms, base + 64 * r + lane, sp, beta1, ob1, acc,
                              word);
        mine = lane == r ? word : mine;
      }
    }
    acc = butterfly(acc);
    if (lane < rows) bits[wbase + lane] = mine;
    if (lane == 0) wpart[((int64_t)w * n + j) * nseg + s] = acc;
  }
}

// ---------------------------------------------------------- scale finalize --
// One block per (worker, chunk) or per chunk: pairwise sum of the segment
// partials (padded with zeros to a power of two), then
// scale = (float)(sqrt(S) / sqrt((double)L)).
constexpr int kGroup = 2 * kBlock;  // partials folded per pass of the block
constexpr int kMaxGroups = 4096;

__global__ void __launch_bounds__(kBlock)
    scale_kernel(const double* __restrict__ part, int64_t nseg, int64_t L, int rows_per_launch,
                 int part_row0, float* __restrict__ scale_out) {
  __shared__ double red[kBlock];
  __shared__ double grpA[kMaxGroups];
  __shared__ double grpB[kMaxGroups / 2];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const double* __restrict__ p = part + (int64_t)(part_row0 + row) * nseg;
  int64_t width = 1;
  while (width < nseg) width <<= 1;
  const int64_t ngroups = width <= kGroup ? 1 : width / kGroup;
  for (int64_t gi = 0; gi < ngroups; ++gi) {
    const int64_t i0 = gi * kGroup + 2 * t;
    const double a = i0 < nseg ? p[i0] : 0.0;
    const double b = i0 + 1 < nseg ? p[i0 + 1] : 0.0;
    red[t] = a + b;
    __syncthreads();
    for (int h = kBlock / 2; h >= 1; h >>= 1) {
      double val = 0.0;
      if (t < h) val = red[2 * t] + red[2 * t + 1];
      __syncthreads();
      if (t < h) red[t] = val;
      __syncthreads();
    }
    if (t == 0) grpA[gi] = red[0];
    __syncthreads();
  }
  // pairwise over the group results (a power of two of them)
  double* src = grpA;
  double* dst = grpB;
  for (int64_t cnt = ngroups; cnt > 1; cnt >>= 1) {
    const int64_t half = cnt >> 1;
    for (int64_t i = t; i < half; i += kBlock) dst[i] = src[2 * i] + src[2 * i + 1];
    __syncthreads();
    double* tmp = src;
    src = dst;
    dst = tmp;
  }
  (void)rows_per_launch;
  if (t == 0) {
    const double S = src[0];
    scale_out[row] = (float)(sqrt(S) / sqrt((double)L));
  }
}

// ------------------------------------------------------------- server pass --
// Server j: a = pairwise over workers of (bit ? s_wj : -s_wj) / n;
// u = a + (u_prev - (u_prev >= 0 ? s_prev : -s_prev)); stores u, sign words,
// segment partials.  grid.y = chunk; grid.x strides over segments.
template <int NW>
__device__ __forceinline__ float worker_average(const uint64_t* __restrict__ wbits, int64_t words,
                                                int64_t row, const float* ws, int n) {
  float vals[NW > 0 ? NW : kMaxWorkersPerLaunch];
  if constexpr (NW > 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w) vals[w] = signed_scale(wbits[(int64_t)w * words + row], ws[w]);
    return pairwise_sum<NW>(vals) / (float)NW;
  } else {
    for (int w = 0; w < n; ++w) vals[w] = signed_scale(wbits[(int64_t)w * words + row], ws[w]);
    return pairwise_sum_any(vals, n) / (float)n;
  }
}

template <int NW>
__global__ void __launch_bounds__(kBlock)
    server_kernel(int64_t L, int n, int64_t nseg, int64_t words,
                  const uint64_t* __restrict__ wbits, const float* __restrict__ wscale,
                  float* __restrict__ u, const float* __restrict__ sscale_prev,
                  uint64_t* __restrict__ sbits, double* __restrict__ spart) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.y;
  float ws[NW > 0 ? NW : kMaxWorkersPerLaunch];
  const int nw = NW > 0 ? NW : n;
#pragma unroll
  for (int w = 0; w < (NW > 0 ? NW : kMaxWorkersPerLaunch); ++w)
    if (w < nw) ws[w] = wscale[w * n + j];
  const float sp = sscale_prev[j];
  const int64_t nwave = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t s = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block(); s < nseg;
       s += nwave) {
    const int64_t q0 = s * kSegElems;
    const int64_t left = (L - q0) >> 6;
    const int rows = left < kSegRows ? (int)left : kSegRows;
    const int64_t base = (int64_t)j * L + q0;
    const int64_t wbase = base >> 6;
    double acc = 0.0;
    uint64_t mine = 0;
    for (int r = 0; r < rows; ++r) {
      const int64_t k = base + 64 * r + lane;
      const float up = u[k];
      const float e = up - (up >= 0.0f ? sp : -sp);
      const float a = worker_average<NW>(wbits, words, wbase + r, ws, n);
      const float uv = a + e;
      u[k] = uv;
      const uint64_t word = __ballot(uv >= 0.0f);
      mine = lane == r ? word : mine;
      acc = add_square(acc, uv);
    }
    acc = butterfly(acc);
    if (lane < rows) sbits[wbase + lane] = mine;
    if (lane == 0) spart[(int64_t)j * nseg + s] = acc;
  }
}

// ------------------------------------------------------------------ update --
// m = (bit ? s_j : -s_j); x = x - lr * (m / (sqrtf(v) + eps)).  A wave owns 16
// consecutive rows of the flat vector; the chunk of a row is row*64 / L.
__global__ void __launch_bounds__(kBlock)
    update_kernel(int64_t words, int64_t L, const uint64_t* __restrict__ sbits,
                  const float* __restrict__ sscale, const float* __restrict__ v,
                  float* __restrict__ x, float lr, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t ngroups = (words + kSegRows - 1) / kSegRows;
  const int64_t nwave = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t rows_per_chunk = L >> 6;
  for (int64_t gi = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block(); gi < ngroups;
       gi += nwave) {
    const int64_t r0 = gi * kSegRows;
    const int rows = words - r0 < kSegRows ? (int)(words - r0) : kSegRows;
    for (int r = 0; r < rows; ++r) {
      const int64_t row = r0 + r;
      const float s = sscale[row / rows_per_chunk];
      const int64_t k = row * 64 + lane;
      const float mv = signed_scale(sbits[row], s);
      x[k] = x[k] - lr * (mv / (sqrtf(v[k]) + eps));
    }
  }
}

// ------------------------------------------------------------- readback ----
__global__ void __launch_bounds__(kBlock)
    error_out_kernel(const float* __restrict__ comp, const float* __restrict__ scales, int64_t L,
                     int64_t offset, int64_t count, float* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count; i += stride) {
    const int64_t k = offset + i;
    const float s = scales[k / L];
    const float cv = comp[k];
    dst[i] = cv - (cv >= 0.0f ? s : -s);
  }
}

__global__ void __launch_bounds__(kBlock)
    decompress_out_kernel(const uint64_t* __restrict__ bits, const float* __restrict__ scales,
                          int64_t L, int64_t offset, int64_t count, float* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count; i += stride) {
    const int64_t k = offset + i;
    const float s = scales[k / L];
    dst[i] = ((bits[k >> 6] >> (k & 63)) & 1u) ? s : -s;
  }
}

unsigned grid_for(int64_t items, int64_t per_block, int64_t cap) {
  int64_t b = (items + per_block - 1) / per_block;
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return (unsigned)b;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

}  // namespace

Layout layout_for(int64_t d, int n) {
  Layout l{};
  const uint64_t ud = (uint64_t)d, un = (uint64_t)n;
  const uint64_t nseg = (uint64_t)((d / n + kSegElems - 1) / kSegElems);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    uint64_t at = off;
    off = align256(off + bytes);
    return at;
  };
  l.x = take(4 * ud);
  l.m = take(4 * ud);
  l.v = take(4 * ud);
  l.u = take(4 * ud);
  l.c = take(4 * ud * un);
  l.wbits = take(8 * (ud / 64) * un);
  l.sbits = take(8 * (ud / 64));
  l.wpart = take(8 * un * un * nseg);
  l.spart = take(8 * un * nseg);
  l.wscale = take(4 * un * un);
  l.sscale = take(4 * un);
  l.total = off;
  return l;
}

hipError_t launch_warmup(const State& s, const GradPtrs& g, float lr, float bc1, float bc2,
                         hipStream_t stream) {
  const float ob1 = 1.0f - s.beta1, ob2 = 1.0f - s.beta2;
  const unsigned grid = grid_for(s.d, kBlock, 8192);
#define OB_WARM(GT, NW)                                                                        \
  warmup_kernel<GT, NW><<<grid, kBlock, 0, stream>>>(g, s.n, s.d, s.m, s.v, s.x, s.beta1, ob1, \
                                                     s.beta2, ob2, bc1, bc2, lr, s.eps)
#define OB_WARM_N(GT)      \
  switch (s.n) {           \
    case 1: OB_WARM(GT, 1); break;   \
    case 2: OB_WARM(GT, 2); break;   \
    case 4: OB_WARM(GT, 4); break;   \
    case 8: OB_WARM(GT, 8); break;   \
    case 16: OB_WARM(GT, 16); break; \
    case 32: OB_WARM(GT, 32); break; \
    case 64: OB_WARM(GT, 64); break; \
    default: OB_WARM(GT, 0); break;  \
  }
  if (s.grad_bf16) {
    OB_WARM_N(uint16_t)
  } else {
    OB_WARM_N(float)
  }
#undef OB_WARM_N
#undef OB_WARM
  return hipGetLastError();
}

hipError_t launch_worker_pass(const State& s, const GradPtrs& g, int w0, int nw, bool m_bits,
                              hipStream_t stream) {
  const float ob1 = 1.0f - s.beta1;
  dim3 grid(grid_for(s.nseg, kWavesPerBlock, 1 << 20), (unsigned)(nw * s.n));
#define OB_WORK(GT, MB)                                                                          \
  worker_kernel<GT, MB><<<grid, kBlock, 0, stream>>>(g, w0, s.d, s.L, s.n, s.nseg, s.words, s.m, \
                                                     s.sbits, s.sscale, s.c, s.wscale, s.wbits,  \
                                                     s.wpart, s.beta1, ob1)
  if (s.grad_bf16) {
    if (m_bits) OB_WORK(uint16_t, true); else OB_WORK(uint16_t, false);
  } else {
    if (m_bits) OB_WORK(float, true); else OB_WORK(float, false);
  }
#undef OB_WORK
  return hipGetLastError();
}

hipError_t launch_worker_scales(const State& s, hipStream_t stream) {
  scale_kernel<<<s.n * s.n, kBlock, 0, stream>>>(s.wpart, s.nseg, s.L, s.n * s.n, 0, s.wscale);
  return hipGetLastError();
}

hipError_t launch_server_pass(const State& s, hipStream_t stream) {
  dim3 grid(grid_for(s.nseg, kWavesPerBlock, 1 << 20), (unsigned)s.n);
#define OB_SRV(NW)                                                                        \
  server_kernel<NW><<<grid, kBlock, 0, stream>>>(s.L, s.n, s.nseg, s.words, s.wbits,      \
                                                 s.wscale, s.u, s.sscale, s.sbits, s.spart)
  switch (s.n) {
    case 1: OB_SRV(1); break;
    case 2: OB_SRV(2); break;
    case 4: OB_SRV(4); break;
    case 8: OB_SRV(8); break;
    case 16: OB_SRV(16); break;
    case 32: OB_SRV(32); break;
    case 64: OB_SRV(64); break;
    default: OB_SRV(0); break;
  }
#undef OB_SRV
  return hipGetLastError();
}

hipError_t launch_server_scales(const State& s, hipStream_t stream) {
  scale_kernel<<<s.n, kBlock, 0, stream>>>(s.spart, s.nseg, s.L, s.n, 0, s.sscale);
  return hipGetLastError();
}

hipError_t launch_update(const State& s, float lr, hipStream_t stream) {
  const int64_t groups = (s.words + kSegRows - 1) / kSegRows;
  update_kernel<<<grid_for(groups, kWavesPerBlock, 1 << 20), kBlock, 0, stream>>>(
      s.words, s.L, s.sbits, s.sscale, s.v, s.x, lr, s.eps);
  return hipGetLastError();
}

hipError_t launch_error_out(const float* comp, const float* scales, int64_t L, int64_t offset,
                            int64_t count, float* dst, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  error_out_kernel<<<grid_for(count, kBlock, 16384), kBlock, 0, stream>>>(comp, scales, L, offset,
                                                                          count, dst);
  return hipGetLastError();
}

hipError_t launch_decompress_out(const uint64_t* bits, const float* scales, int64_t L,
                                 int64_t offset, int64_t count, float* dst, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  decompress_out_kernel<<<grid_for(count, kBlock, 16384), kBlock, 0, stream>>>(bits, scales, L,
                                                                               offset, count, dst);
  return hipGetLastError();
}

}  // namespace ob
