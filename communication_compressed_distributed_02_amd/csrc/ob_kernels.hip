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
//  - The momentum's sign words are read with scalar (uniform) loads and
//    decoded with an inverse ballot: bit `lane` of a uniform 64-bit word
//    selects +s or -s in one v_cndmask.
//  - The worker grid is non-persistent (one wave per segment, grid.y =
//    worker x chunk): persistent grids and several segments per wave
//    measured slower.
//  - The server pass for 8 to 64 workers looks up sums of 4-worker subtrees
//    in LDS tables, indexed by the sign bits that a cross-lane bit transpose
//    of vector-loaded sign words puts in each lane; for other worker counts
//    it folds the workers' +-s in worker order into per-row stacks.  Both
//    reproduce the pairwise-by-levels sum exactly.
//  - The worker and server passes fold the partials of a block's 4 aligned
//    segments in LDS (the first two levels of the pairwise tree over a
//    chunk's segment partials), so they write one partial per block; the
//    server pass for 32 and 64 workers writes one per segment.
//  - Where chunks have an even number of rows, the server pass copies each
//    segment's sign words of all workers whole into LDS with gfx950's direct
//    global-to-LDS loads, so each worker's 128-byte line is fetched once.
//  - A streaming pass over more than 2^26 elements is issued as a sequence of
//    launches of about that size (launch_parts): on MI355X that moves more
//    bytes per second than one launch over billions of elements.
//  - Per-chunk scales come from small kernels: one dispatch that folds a
//    chunk's partials in registers and one block, or aligned groups of 512
//    partials folded in parallel and then one block per chunk.  Where the
//    rows of partials are short (at most 64, as on 1M-parameter shapes),
//    the passes that need the scales fold them themselves -- every server
//    block its chunk's worker rows, every update block the server rows -- in
//    the same order, and a step is three dispatches.
#include <algorithm>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ob_kernels.h"

namespace ob {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int64_t kMaxBlocksPerRow = int64_t(1) << 20;
static_assert(kWavesPerBlock == 4, "the worker pass folds 4 segment partials per block");

// Blocks of 4 aligned segments in a chunk of nseg segments.
__host__ __device__ constexpr int64_t quads(int64_t nseg) {
  return (nseg + kWavesPerBlock - 1) / kWavesPerBlock;
}

// The part of a pass's grid that one launch covers: block (x, y) of the
// launch is block (bx0 + x, by0 + y) of the whole pass.  The update, whose
// waves stride over groups of 16 rows, takes the groups [lo, hi) instead.
struct Part {
  int64_t bx0;
  int by0;
  int64_t lo, hi;
};

// The server pass for 32 and 64 workers leaves one partial per segment; every
// other pass leaves one per block of 4 segments.
constexpr bool server_segment_partials(int n) { return n == 32 || n == 64; }

// Streamed (read-once / write-once per step) accesses are non-temporal: the
// step's working set is many times the caches, so nothing streamed is reused
// before eviction (worker pass 1.94 -> 1.48 ms on 110M x 8 workers).
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) { __builtin_nontemporal_store(v, p); }

// Index of this wavefront in its block, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ float grad_value(const float* g, int64_t k) { return ld_stream(g + k); }
__device__ __forceinline__ float grad_value(const uint16_t* g, int64_t k) {
  return __uint_as_float((uint32_t)ld_stream(g + k) << 16);  // bf16 -> fp32, exact
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

// The partials of a block's 4 aligned segments (wave w's `acc`; 0 for a
// segment past the chunk's end, like the zero padding) folded as
// ((p0 + p1) + (p2 + p3)) -- the first two levels of the pairwise sum over
// a chunk's segment partials -- and stored at *dst.  Every thread of the
// block must reach it (it holds two barriers).
__device__ __forceinline__ void store_quad_partial(double acc, double* quad_part, double* dst) {
  if ((threadIdx.x & 63) == 0) quad_part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) *dst = (quad_part[0] + quad_part[1]) + (quad_part[2] + quad_part[3]);
  __syncthreads();
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

// Pairwise sum by levels of value(0), ..., value(n-1) for any 1 <= n <= 64
// (an odd tail passes up), in registers.  The values are pushed into a
// binary-counter stack: level l holds the sum of an aligned block of 2^l
// values, and value w merges the levels given by the trailing one bits of w
// (stack level + carry).  The levels left at the end are the set bits of n;
// folding them from the lowest up (higher level + carry) completes exactly
// the pairwise-by-levels tree.  Levels are compile-time indices, so nothing
// goes to scratch memory.
constexpr int kStackLevels = 7;  // floor(log2(64)) + 1

template <typename F>
__device__ __forceinline__ float pairwise_sum_stream(int n, F value) {
  float stack[kStackLevels];
  for (int w = 0; w < n; ++w) {
    float v = value(w);
    int x = w;
    bool carry = true;
#pragma unroll
    for (int l = 0; l < kStackLevels; ++l) {
      if (carry) {
        if (x & 1) {
          v = stack[l] + v;
          x >>= 1;
        } else {
          stack[l] = v;
          carry = false;
        }
      }
    }
  }
  float acc = 0.0f;
  bool have = false;
#pragma unroll
  for (int l = 0; l < kStackLevels; ++l) {
    if ((n >> l) & 1) {
      acc = have ? stack[l] + acc : stack[l];
      have = true;
    }
  }
  return acc;
}

// ----------------------------------------------------------------- warm-up --
// Full-precision Adam with bias correction on the pairwise worker average.
__device__ __forceinline__ void adam_element(float gbar, float& m, float& v, float& x,
                                             float beta1, float ob1, float beta2, float ob2,
                                             float bc1, float bc2, float lr, float eps) {
  m = (beta1 * m) + (ob1 * gbar);
  v = (beta2 * v) + (ob2 * (gbar * gbar));
  const float mh = m / bc1;
  const float vh = v / bc2;
  x = x - lr * (mh / (sqrtf(vh) + eps));
}

// NW a power of two: a wave owns R consecutive rows of 64 at a time (R = 4,
// 2, 1 as NW grows, so the NW*R gradient registers stay bounded), issues all
// loads of those rows first and streams them non-temporally.
template <typename GT, int NW>
__global__ void __launch_bounds__(kBlock)
    warmup_rows_kernel(GradPtrs g, int64_t words, float* __restrict__ m, float* __restrict__ v,
                       float* __restrict__ x, float beta1, float ob1, float beta2, float ob2,
                       float bc1, float bc2, float lr, float eps) {
  constexpr int R = NW <= 8 ? 4 : (NW <= 16 ? 2 : 1);
  const int lane = threadIdx.x & 63;
  const int64_t ngroups = words / R;  // full groups; a tail of rows is handled below
  const int64_t nwave = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t first = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  for (int64_t gi = first; gi < ngroups; gi += nwave) {
    const int64_t k0 = gi * R * 64 + lane;
    float gv[R][NW], mv[R], vv[R], xv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int w = 0; w < NW; ++w) gv[r][w] = grad_value((const GT*)g.p[w], k0 + 64 * r);
      mv[r] = ld_stream(m + k0 + 64 * r);
      vv[r] = ld_stream(v + k0 + 64 * r);
      xv[r] = ld_stream(x + k0 + 64 * r);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float gbar = pairwise_sum<NW>(gv[r]) / (float)NW;
      adam_element(gbar, mv[r], vv[r], xv[r], beta1, ob1, beta2, ob2, bc1, bc2, lr, eps);
      st_stream(m + k0 + 64 * r, mv[r]);
      st_stream(v + k0 + 64 * r, vv[r]);
      st_stream(x + k0 + 64 * r, xv[r]);
    }
  }
  // rows past the last full group: one row per wave
  for (int64_t row = ngroups * R + first; row < words; row += nwave) {
    const int64_t k = row * 64 + lane;
    float vals[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) vals[w] = grad_value((const GT*)g.p[w], k);
    const float gbar = pairwise_sum<NW>(vals) / (float)NW;
    float mk = m[k], vk = v[k], xk = x[k];
    adam_element(gbar, mk, vk, xk, beta1, ob1, beta2, ob2, bc1, bc2, lr, eps);
    m[k] = mk;
    v[k] = vk;
    x[k] = xk;
  }
}

// Worker-at-a-time warm-up.  The gradients are summed in the pairwise order
// by a binary-counter stack of partial sums, level l at stack + l*d: worker w
// merges the levels 0..merges-1 (merges = trailing one bits of w), each as
// (stack level) + (carry), and leaves its carry at level `merges`.  After all n
// workers the occupied levels are the set bits of n; folding them from the
// lowest level up, each as (higher level) + (carry), is exactly the
// pairwise-by-levels sum with odd tails passing up.
template <typename GT>
__global__ void __launch_bounds__(kBlock)
    warmup_push_kernel(const GT* __restrict__ g, float* __restrict__ stack, int64_t d,
                       int merges) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < d; k += stride) {
    float v = grad_value(g, k);
    for (int l = 0; l < merges; ++l) v = ld_stream(stack + (int64_t)l * d + k) + v;
    st_stream(stack + (int64_t)merges * d + k, v);
  }
}

// Fold the stack, average, one Adam step; then clear every stack level used
// (levels 0..levels-1), so the slabs hold zeros again.
__global__ void __launch_bounds__(kBlock)
    warmup_finish_kernel(float* __restrict__ stack, int64_t d, int n, int levels,
                         float* __restrict__ m, float* __restrict__ v, float* __restrict__ x,
                         float beta1, float ob1, float beta2, float ob2, float bc1, float bc2,
                         float lr, float eps) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < d; k += stride) {
    float acc = 0.0f;
    bool have = false;
    for (int l = 0; l < levels; ++l) {
      if ((n >> l) & 1) {
        const float s = ld_stream(stack + (int64_t)l * d + k);
        acc = have ? s + acc : s;
        have = true;
      }
    }
    const float gbar = acc / (float)n;
    float mk = m[k], vk = v[k], xk = x[k];
    adam_element(gbar, mk, vk, xk, beta1, ob1, beta2, ob2, bc1, bc2, lr, eps);
    m[k] = mk;
    v[k] = vk;
    x[k] = xk;
    for (int l = 0; l < levels; ++l) st_stream(stack + (int64_t)l * d + k, 0.0f);
  }
}

// Any n <= 64 (run-time count, pairwise with odd tails): one element per thread.
template <typename GT, int NW>
__global__ void __launch_bounds__(kBlock)
    warmup_kernel(GradPtrs g, int n, int64_t d, float* __restrict__ m, float* __restrict__ v,
                  float* __restrict__ x, float beta1, float ob1, float beta2, float ob2, float bc1,
                  float bc2, float lr, float eps) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < d; k += stride) {
    float sum;
    if constexpr (NW > 0) {
      float vals[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) vals[w] = grad_value((const GT*)g.p[w], k);
      sum = pairwise_sum<NW>(vals);
    } else {
      sum = pairwise_sum_stream(n, [&](int w) { return grad_value((const GT*)g.p[w], k); });
    }
    const float gbar = sum / (float)(NW > 0 ? NW : n);
    float mk = m[k], vk = v[k], xk = x[k];
    adam_element(gbar, mk, vk, xk, beta1, ob1, beta2, ob2, bc1, bc2, lr, eps);
    m[k] = mk;
    v[k] = vk;
    x[k] = xk;
  }
}

// ------------------------------------------------------------- worker pass --
// c = ((b1*m) + ((1-b1)*g)) + e with e = c_prev - (c_prev >= 0 ? s_prev : -s_prev);
// stores c, the row's sign word and the segment's fp64 sum of squares.
// grid.y = (worker in launch) * n + chunk; grid.x strides over segments.
// bm = b1*m, formed by the caller.
template <typename GT>
__device__ __forceinline__ void worker_row(const GT* __restrict__ g, float* __restrict__ c,
                                           float bm, int64_t k, float sp, float ob1,
                                           double& acc, uint64_t& word) {
  const float gv = grad_value(g, k);
  const float cp = ld_stream(c + k);
  const float e = cp - (cp >= 0.0f ? sp : -sp);
  const float cv = (bm + (ob1 * gv)) + e;
  st_stream(c + k, cv);
  word = __ballot(cv >= 0.0f);
  acc = add_square(acc, cv);
}

// The block's 4 waves own 4 consecutive segments, aligned at a multiple of 4,
// and their partials are folded in LDS (store_quad_partial), so one fp64
// partial per block reaches HBM and the finalize folds 4x fewer.  One block
// per quad (grid.x == quads(nseg)): a grid-stride loop here, never taken
// twice, held 42-50 VGPRs against 32-37 without it.  The momentum is the
// server's sign words and scales of the previous step.
template <typename GT>
__global__ void __launch_bounds__(kBlock)
    worker_kernel(GradPtrs g, int w0, Part pt, int64_t d, int64_t L, int n, int64_t nseg, int64_t words,
                  const uint64_t* __restrict__ sbits, const float* __restrict__ sscale,
                  float* __restrict__ cbuf, const float* __restrict__ wscale,
                  uint64_t* __restrict__ wbits, double* __restrict__ wpart, float beta1,
                  float ob1) {
  __shared__ double quad_part[kWavesPerBlock];
  const int lane = threadIdx.x & 63;
  const int wv = wave_in_block();
  const int y = pt.by0 + (int)blockIdx.y;
  const int wi = y / n;  // worker within this pass
  const int j = y - wi * n;
  const int w = w0 + wi;
  const GT* __restrict__ gp = (const GT*)g.p[wi];
  float* __restrict__ c = cbuf + (int64_t)w * d;
  uint64_t* __restrict__ bits = wbits + (int64_t)w * words;
  const int64_t nquad = quads(nseg);
  double* __restrict__ part = wpart + ((int64_t)w * n + j) * nquad;
  const float sp = wscale[w * n + j];  // this worker's scale of chunk j, previous step
  const float ms = sscale[j];
  {
    const int64_t qd = pt.bx0 + blockIdx.x;  // one quad per block
    const int64_t s = qd * kWavesPerBlock + wv;
    double acc = 0.0;
    if (s < nseg) {
      const int64_t q0 = s * kSegElems;
      const int64_t left = (L - q0) >> 6;
      const int rows = left < kSegRows ? (int)left : kSegRows;
      const int64_t base = (int64_t)j * L + q0;  // global index of the segment's first element
      const int64_t wbase = base >> 6;
      uint64_t mine = 0;
      if (rows == kSegRows) {
        // fully unrolled: the compiler keeps 16 of the segment's 32 loads in
        // flight and issues the others as registers free (all 32 first, at
        // 66 VGPRs, measured no faster)
#pragma unroll
        for (int r = 0; r < kSegRows; ++r) {
          uint64_t word;
          worker_row<GT>(gp, c, beta1 * signed_scale(sbits[wbase + r], ms), base + 64 * r + lane,
                         sp, ob1, acc, word);
          mine = lane == r ? word : mine;
        }
      } else {
        for (int r = 0; r < rows; ++r) {
          uint64_t word;
          worker_row<GT>(gp, c, beta1 * signed_scale(sbits[wbase + r], ms), base + 64 * r + lane,
                         sp, ob1, acc, word);
          mine = lane == r ? word : mine;
        }
      }
      acc = butterfly(acc);
      if (lane < rows) bits[wbase + lane] = mine;
    }
    store_quad_partial(acc, quad_part, part + qd);
  }
}

// bm[r] = b1 * m[k0 + 64*r] for the rows of a segment, all loads issued
// before the first use (compile-time indices only, so bm lives in
// registers).  A ragged segment's missing rows load its last row again
// (unused) rather than branch per row, which made every load wait for the
// one before it; a wave past the chunk's end (rows == 0) loads nothing.
__device__ __forceinline__ void load_bm(float* bm, const float* __restrict__ m, int64_t k0,
                                        int rows, float beta1) {
  if (rows == 0) return;
#pragma unroll
  for (int r = 0; r < kSegRows; ++r)
    bm[r] = beta1 * ld_stream(m + k0 + 64 * (r < rows ? r : rows - 1));
}

// The first compressed step, where the momentum is still the warm-up's fp32
// m.  A block runs its quad for `wg` consecutive workers of the launch in
// turn (grid.y = worker group * n + chunk): a wave reads its segment of m
// once and keeps b1*m in registers, so m is read once per group instead of
// once per worker.  Each worker's values, sign words and partials are those
// of worker_kernel (the same fp32 operations per element, the same order of
// sums).
template <typename GT>
__global__ void __launch_bounds__(kBlock)
    worker_first_kernel(GradPtrs g, int w0, int wg, Part pt, int64_t d, int64_t L, int n,
                        int64_t nseg, int64_t words, const float* __restrict__ m,
                        float* __restrict__ cbuf, const float* __restrict__ wscale,
                        uint64_t* __restrict__ wbits, double* __restrict__ wpart, float beta1,
                        float ob1) {
  __shared__ double quad_part[kWavesPerBlock];
  const int lane = threadIdx.x & 63;
  const int wv = wave_in_block();
  const int y = pt.by0 + (int)blockIdx.y;
  const int wg0 = (y / n) * wg;  // the group's first worker within the launch
  const int j = y - (y / n) * n;
  const int64_t nquad = quads(nseg);
  const int64_t qd = pt.bx0 + blockIdx.x;  // one quad per block
  const int64_t s = qd * kWavesPerBlock + wv;
  const bool live = s < nseg;
  const int64_t q0 = s * kSegElems;
  const int64_t left = live ? (L - q0) >> 6 : 0;
  const int rows = left < kSegRows ? (int)left : kSegRows;
  const int64_t base = (int64_t)j * L + q0;
  const int64_t wbase = base >> 6;
  float bm[kSegRows];
  load_bm(bm, m, base + lane, rows, beta1);
  for (int wi = wg0; wi < wg0 + wg; ++wi) {
    const int w = w0 + wi;
    const GT* __restrict__ gp = (const GT*)g.p[wi];
    float* __restrict__ c = cbuf + (int64_t)w * d;
    const float sp = wscale[w * n + j];
    double acc = 0.0;
    if (live) {
      uint64_t mine = 0;
      if (rows == kSegRows) {
#pragma unroll
        for (int r = 0; r < kSegRows; ++r) {
          uint64_t word;
          worker_row<GT>(gp, c, bm[r], base + 64 * r + lane, sp, ob1, acc, word);
          mine = lane == r ? word : mine;
        }
      } else {
#pragma unroll
        for (int r = 0; r < kSegRows; ++r) {
          if (r < rows) {
            uint64_t word;
            worker_row<GT>(gp, c, bm[r], base + 64 * r + lane, sp, ob1, acc, word);
            mine = lane == r ? word : mine;
          }
        }
      }
      acc = butterfly(acc);
      if (lane < rows) wbits[(int64_t)w * words + wbase + lane] = mine;
    }
    store_quad_partial(acc, quad_part, wpart + ((int64_t)w * n + j) * nquad + qd);
  }
}

// ------------------------------------------------------------ 0/1 Adam --
// "Maximizing Communication Efficiency for Large-scale Training via 0/1
// Adam" (abstract): local momentum steps with a stale variance, their
// step-weighted mean momentum sent through the same 1-bit codec at a
// synchronization.  Per worker and element, a local step is
//   m_i = (b1*m_src) + ((1-b1)*g_i),   m_src = shared m at the first step of
//                                      a period, m_i afterwards;
//   a_i = m_i at the first step, a_i + (w*(m_i - a_i)) afterwards, w = lr/G
//         (G = the period's summed step sizes, formed on the host);
// a synchronizing step then forms c = a_i + e_i and compresses it exactly as
// the worker pass does.  Same mapping as the worker pass (one wave per
// segment of a (worker, chunk) row, grid.y = worker * n + chunk).

template <typename GT, bool FIRST, bool MBITS>
__device__ __forceinline__ void zo_momentum(const GT* __restrict__ g, const float* __restrict__ m,
                                            const float* __restrict__ mloc,
                                            const float* __restrict__ aloc, uint64_t mword,
                                            float ms, int64_t k, float beta1, float ob1, float wk,
                                            float& mi, float& ai) {
  const float gv = grad_value(g, k);
  const float msrc = FIRST ? (MBITS ? signed_scale(mword, ms) : m[k]) : ld_stream(mloc + k);
  mi = (beta1 * msrc) + (ob1 * gv);
  if (FIRST) {
    ai = mi;
  } else {
    const float ap = ld_stream(aloc + k);
    ai = ap + (wk * (mi - ap));
  }
}

// A local step (no synchronization): stores m_i and a_i.
template <typename GT, bool FIRST, bool MBITS>
__global__ void __launch_bounds__(kBlock)
    zo_local_kernel(GradPtrs g, Part pt, int64_t d, int64_t L, int n, int64_t nseg,
                    const float* __restrict__ m, const uint64_t* __restrict__ sbits,
                    const float* __restrict__ sscale, float* __restrict__ mlocbuf,
                    float* __restrict__ alocbuf, float beta1, float ob1, float wk) {
  const int lane = threadIdx.x & 63;
  const int y = pt.by0 + (int)blockIdx.y;
  const int wi = y / n;
  const int j = y - wi * n;
  const GT* __restrict__ gp = (const GT*)g.p[wi];
  float* __restrict__ mloc = mlocbuf + (int64_t)wi * d;
  float* __restrict__ aloc = alocbuf + (int64_t)wi * d;
  const float ms = MBITS ? sscale[j] : 0.0f;
  const int64_t s = (pt.bx0 + (int64_t)blockIdx.x) * kWavesPerBlock + wave_in_block();
  if (s >= nseg) return;
  const int64_t q0 = s * kSegElems;
  const int64_t left = (L - q0) >> 6;
  const int rows = left < kSegRows ? (int)left : kSegRows;
  const int64_t base = (int64_t)j * L + q0;
  const int64_t wbase = base >> 6;
  if (rows == kSegRows) {
#pragma unroll
    for (int r = 0; r < kSegRows; ++r) {
      const int64_t k = base + 64 * r + lane;
      float mi, ai;
      zo_momentum<GT, FIRST, MBITS>(gp, m, mloc, aloc, MBITS ? sbits[wbase + r] : 0, ms, k,
                                    beta1, ob1, wk, mi, ai);
      st_stream(mloc + k, mi);
      st_stream(aloc + k, ai);
    }
  } else {
    for (int r = 0; r < rows; ++r) {
      const int64_t k = base + 64 * r + lane;
      float mi, ai;
      zo_momentum<GT, FIRST, MBITS>(gp, m, mloc, aloc, MBITS ? sbits[wbase + r] : 0, ms, k,
                                    beta1, ob1, wk, mi, ai);
      st_stream(mloc + k, mi);
      st_stream(aloc + k, ai);
    }
  }
}

// The first local step after the warm-up, where the shared momentum is still
// the warm-up's fp32 m: as worker_first_kernel, a wave reads its segment of m
// once and runs the local step of that segment for the `wg` workers of its
// group in turn (m_i = a_i = (b1*m) + ((1-b1)*g_i), the same fp32 operations
// as zo_local_kernel).  grid.y = worker group * n + chunk.
template <typename GT>
__global__ void __launch_bounds__(kBlock)
    zo_local_first_kernel(GradPtrs g, int wg, Part pt, int64_t d, int64_t L, int n,
                          int64_t nseg, const float* __restrict__ m, float* __restrict__ mlocbuf,
                          float* __restrict__ alocbuf, float beta1, float ob1) {
  const int lane = threadIdx.x & 63;
  const int y = pt.by0 + (int)blockIdx.y;
  const int wg0 = (y / n) * wg;
  const int j = y - (y / n) * n;
  const int64_t s = (pt.bx0 + (int64_t)blockIdx.x) * kWavesPerBlock + wave_in_block();
  if (s >= nseg) return;
  const int64_t q0 = s * kSegElems;
  const int64_t left = (L - q0) >> 6;
  const int rows = left < kSegRows ? (int)left : kSegRows;
  const int64_t base = (int64_t)j * L + q0;
  float bm[kSegRows];
  load_bm(bm, m, base + lane, rows, beta1);
  for (int wi = wg0; wi < wg0 + wg; ++wi) {
    const GT* __restrict__ gp = (const GT*)g.p[wi];
    float* __restrict__ mloc = mlocbuf + (int64_t)wi * d;
    float* __restrict__ aloc = alocbuf + (int64_t)wi * d;
    auto row = [&](int r) {
      const int64_t k = base + 64 * r + lane;
      const float mi = bm[r] + (ob1 * grad_value(gp, k));
      st_stream(mloc + k, mi);
      st_stream(aloc + k, mi);
    };
    if (rows == kSegRows) {
#pragma unroll
      for (int r = 0; r < kSegRows; ++r) row(r);
    } else {
#pragma unroll
      for (int r = 0; r < kSegRows; ++r)
        if (r < rows) row(r);
    }
  }
}

// A synchronizing step's worker pass: the local step's a_i (not stored: the
// period ends), then c = a_i + e with e = c_prev - (c_prev >= 0 ? s_prev :
// -s_prev), stored with its sign words and the block's partial of the sum of
// squares, as in worker_kernel.
template <typename GT, bool FIRST, bool MBITS>
__global__ void __launch_bounds__(kBlock)
    zo_sync_kernel(GradPtrs g, Part pt, int64_t d, int64_t L, int n, int64_t nseg, int64_t words,
                   const float* __restrict__ m, const uint64_t* __restrict__ sbits,
                   const float* __restrict__ sscale, const float* __restrict__ mlocbuf,
                   const float* __restrict__ alocbuf, float* __restrict__ cbuf,
                   const float* __restrict__ wscale, uint64_t* __restrict__ wbits,
                   double* __restrict__ wpart, float beta1, float ob1, float wk) {
  __shared__ double quad_part[kWavesPerBlock];
  const int lane = threadIdx.x & 63;
  const int wv = wave_in_block();
  const int y = pt.by0 + (int)blockIdx.y;
  const int w = y / n;
  const int j = y - w * n;
  const GT* __restrict__ gp = (const GT*)g.p[w];
  const float* __restrict__ mloc = mlocbuf + (int64_t)w * d;
  const float* __restrict__ aloc = alocbuf + (int64_t)w * d;
  float* __restrict__ c = cbuf + (int64_t)w * d;
  uint64_t* __restrict__ bits = wbits + (int64_t)w * words;
  const int64_t nquad = quads(nseg);
  double* __restrict__ part = wpart + ((int64_t)w * n + j) * nquad;
  const float sp = wscale[w * n + j];  // this worker's scale of chunk j at the last sync
  const float ms = MBITS ? sscale[j] : 0.0f;
  const int64_t qd = pt.bx0 + blockIdx.x;  // one quad per block
  const int64_t s = qd * kWavesPerBlock + wv;
  double acc = 0.0;
  if (s < nseg) {
    const int64_t q0 = s * kSegElems;
    const int64_t left = (L - q0) >> 6;
    const int rows = left < kSegRows ? (int)left : kSegRows;
    const int64_t base = (int64_t)j * L + q0;
    const int64_t wbase = base >> 6;
    uint64_t mine = 0;
    auto row = [&](int r) {
      const int64_t k = base + 64 * r + lane;
      float mi, ai;
      zo_momentum<GT, FIRST, MBITS>(gp, m, mloc, aloc, MBITS ? sbits[wbase + r] : 0, ms, k,
                                    beta1, ob1, wk, mi, ai);
      const float cp = ld_stream(c + k);
      const float cv = ai + (cp - (cp >= 0.0f ? sp : -sp));
      st_stream(c + k, cv);
      const uint64_t word = __ballot(cv >= 0.0f);
      mine = lane == r ? word : mine;
      acc = add_square(acc, cv);
    };
    if (rows == kSegRows) {
#pragma unroll
      for (int r = 0; r < kSegRows; ++r) row(r);
    } else {
      for (int r = 0; r < rows; ++r) row(r);
    }
    acc = butterfly(acc);
    if (lane < rows) bits[wbase + lane] = mine;
  }
  store_quad_partial(acc, quad_part, part + qd);
}

// Variance refresh at a synchronization (after the update, which used the
// stale variance): v = (b2*v) + ((1-b2)*(gbar*gbar)), gbar the pairwise
// worker average of this step's gradients (as in the warm-up).
template <typename GT, int NW>
__global__ void __launch_bounds__(kBlock)
    zo_refresh_kernel(GradPtrs g, int n, int64_t d, float* __restrict__ v, float beta2,
                      float ob2) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < d; k += stride) {
    float sum;
    if constexpr (NW > 0) {
      float vals[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) vals[w] = grad_value((const GT*)g.p[w], k);
      sum = pairwise_sum<NW>(vals);
    } else {
      sum = pairwise_sum_stream(n, [&](int w) { return grad_value((const GT*)g.p[w], k); });
    }
    const float gbar = sum / (float)(NW > 0 ? NW : n);
    v[k] = (beta2 * v[k]) + (ob2 * (gbar * gbar));
  }
}

// ---------------------------------------------------------- scale finalize --
// The pairwise sum over a row's segment partials (padded with zeros to a
// power of two, width W) is split at aligned subtrees of kGroup = 512
// partials: phase 1 folds every group in parallel (grid = groups x rows),
// phase 2 folds a row's group results (a power of two of them) and forms
// scale = (float)(sqrt(S) / sqrt((double)L)).  Zero padding contributes +0
// to every sum it enters, so padding a short row up to one whole group gives
// the same value as its own power-of-two width.
constexpr int kGroup = 2 * kBlock;

// Group results per row of nseg partials (0 when one block folds the row).
int64_t fold_doubles_per_row(int64_t nseg) {
  int64_t width = 1;
  while (width < nseg) width <<= 1;
  return width <= kGroup ? 0 : width / kGroup;
}
static_assert(quads(kMaxSegsPerChunk) <= (int64_t)kGroup * kGroup &&
                  kMaxSegsPerChunkSegPartials <= (int64_t)kGroup * kGroup,
              "one level of group folds leaves at most kGroup values per row");
static_assert(quads(kMaxSegsPerChunk) <= kMaxBlocksPerRow,
              "the worker and server passes launch one block per quad of a row");

// Pairwise fold of the 2*kBlock values a[t], b[t] (t = thread) held as pairs
// (a[t] = element 2t, b[t] = element 2t+1); returns the sum in thread 0.
__device__ double block_pairwise(double a, double b, double* red) {
  const int t = threadIdx.x;
  red[t] = a + b;
  __syncthreads();
  for (int h = kBlock / 2; h >= 1; h >>= 1) {
    double val = 0.0;
    if (t < h) val = red[2 * t] + red[2 * t + 1];
    __syncthreads();
    if (t < h) red[t] = val;
    __syncthreads();
  }
  return red[0];
}

__global__ void __launch_bounds__(kBlock)
    fold_groups_kernel(const double* __restrict__ part, int64_t nseg, int64_t ngroups,
                       double* __restrict__ out) {
  __shared__ double red[kBlock];
  const int t = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t row = blockIdx.y;
  const double* __restrict__ p = part + row * nseg;
  const int64_t i0 = g * kGroup + 2 * t;
  const double a = i0 < nseg ? p[i0] : 0.0;
  const double b = i0 + 1 < nseg ? p[i0 + 1] : 0.0;
  const double sum = block_pairwise(a, b, red);
  if (t == 0) out[row * ngroups + g] = sum;
}

__global__ void __launch_bounds__(kBlock)
    scale_kernel(const double* __restrict__ vals, int64_t count, int64_t L,
                 float* __restrict__ scale_out) {
  // count <= kGroup values per row, zero padded to kGroup
  __shared__ double red[kBlock];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const double* __restrict__ p = vals + row * count;
  const int64_t i0 = 2 * t;
  const double a = i0 < count ? p[i0] : 0.0;
  const double b = i0 + 1 < count ? p[i0 + 1] : 0.0;
  const double S = block_pairwise(a, b, red);
  if (t == 0) scale_out[row] = (float)(sqrt(S) / sqrt((double)L));
}

// Rows of at most kBlock * PER partials in one dispatch: thread t folds the
// aligned run [PER*t, PER*t + PER) pairwise in registers (zeros past the
// row), then the block folds the kBlock run sums pairwise -- the same tree as
// the pairwise sum over the row padded to kBlock * PER.
template <int PER>
__global__ void __launch_bounds__(kBlock)
    scale_direct_kernel(const double* __restrict__ part, int64_t nseg, int64_t L,
                        float* __restrict__ scale_out) {
  __shared__ double red[kBlock];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const double* __restrict__ p = part + row * nseg;
  double v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t k = (int64_t)t * PER + i;
    v[i] = k < nseg ? p[k] : 0.0;
  }
#pragma unroll
  for (int h = PER / 2; h >= 1; h /= 2) {
#pragma unroll
    for (int i = 0; i < h; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  }
  red[t] = v[0];
  __syncthreads();
  for (int h = kBlock / 2; h >= 1; h >>= 1) {
    double val = 0.0;
    if (t < h) val = red[2 * t] + red[2 * t + 1];
    __syncthreads();
    if (t < h) red[t] = val;
    __syncthreads();
  }
  if (t == 0) {
    const double S = red[0];
    scale_out[row] = (float)(sqrt(S) / sqrt((double)L));
  }
}

// Scale of one chunk from a row of `count` <= 64 partials, by one wave:
// lane t takes partial t (+0 past the row, as the finalize kernels pad), and
// an xor butterfly over offsets 1, 2, ..., 32 adds sibling subtrees level by
// level.  IEEE addition commutes, so every lane ends with the row's
// pairwise-by-levels sum, the value the finalize kernels fold, and the scale
// is formed as they form it.
__device__ __forceinline__ float row_scale_wave(const double* __restrict__ p, int64_t count,
                                                int64_t L, int lane) {
  double v = lane < count ? p[lane] : 0.0;
#pragma unroll
  for (int o = 1; o <= 32; o <<= 1) v = v + __shfl_xor(v, o, 64);
  return (float)(sqrt(v) / sqrt((double)L));
}

// Scales of `rows` chunks folded inside a consuming pass: row r's `count`
// <= 64 partials start at part + r*pstride, one wave per row.  They go to
// lds[r] (visible to the whole block after the barrier) and, when `store`
// (one block per set of rows), to out[r*ostride], where the next step's
// passes and the state readback find them.  Every thread of the block must
// reach it.
__device__ __forceinline__ void fold_scales_in_block(const double* __restrict__ part,
                                                     int64_t pstride, int64_t count, int rows,
                                                     int64_t L, float* lds,
                                                     float* __restrict__ out, int64_t ostride,
                                                     bool store) {
  const int lane = threadIdx.x & 63;
  for (int r = wave_in_block(); r < rows; r += kWavesPerBlock) {
    const float sc = row_scale_wave(part + r * pstride, count, L, lane);
    if (lane == 0) {
      lds[r] = sc;
      if (store) out[r * ostride] = sc;
    }
  }
  __syncthreads();
}

// A uniform copy of an LDS value (kept in a scalar register).
__device__ __forceinline__ float uniform_f32(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// ------------------------------------------------------------- server pass --
// Server j: a = pairwise over workers of (bit ? s_wj : -s_wj) / n;
// u = a + (u_prev - (u_prev >= 0 ? s_prev : -s_prev)); stores u, sign words,
// segment partials.  grid.y = chunk; grid.x strides over segments.
//
// Two forms: few workers (n = 1, 2, 4, or a count that is not a power of
// two) read the sign words as uniform scalar loads and select +-s per worker;
// n = 8, 16, 32, 64 use the group tables below.

template <int NW>
__device__ __forceinline__ float worker_average(const uint64_t* __restrict__ wbits, int64_t words,
                                                int64_t row, const float* ws, int n) {
  if constexpr (NW > 0) {
    float vals[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) vals[w] = signed_scale(wbits[(int64_t)w * words + row], ws[w]);
    return pairwise_sum<NW>(vals) / (float)NW;
  } else {
    return pairwise_sum_stream(
               n, [&](int w) { return signed_scale(wbits[(int64_t)w * words + row], ws[w]); }) /
           (float)n;
  }
}

// Full segment, NW = 1, 2 or 4: the 16 sign words of one worker are one
// uniform 128-byte burst; workers are folded into per-row stacks in worker
// order so that the result is exactly the pairwise-by-levels sum (merging
// level l whenever bit l of the worker index is set, left operand first).
template <int NW>
__device__ __forceinline__ void server_average_segment(const uint64_t* __restrict__ wbits,
                                                       int64_t words, int64_t wbase,
                                                       const float* ws, float* avg) {
  constexpr int LEVELS = NW == 1 ? 1 : (NW == 2 ? 2 : 3);
  static_assert(NW == 1 || NW == 2 || NW == 4, "few-worker path");
  float stack[LEVELS][kSegRows];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint64_t* __restrict__ wp = wbits + (int64_t)w * words + wbase;
    float v[kSegRows];
#pragma unroll
    for (int r = 0; r < kSegRows; ++r) v[r] = signed_scale(wp[r], ws[w]);
    int lvl = 0;
#pragma unroll
    for (int x = w; x & 1; x >>= 1, ++lvl) {
#pragma unroll
      for (int r = 0; r < kSegRows; ++r) v[r] = stack[lvl][r] + v[r];
    }
#pragma unroll
    for (int r = 0; r < kSegRows; ++r) stack[lvl][r] = v[r];
  }
#pragma unroll
  for (int r = 0; r < kSegRows; ++r) avg[r] = stack[LEVELS - 1][r] / (float)NW;
}

// NW = 1, 2, 4, or 0 for a run-time worker count.  FOLD: the worker scales
// of chunk j are folded here from the worker pass's partials (`wcount` per
// row), and the chunk's first block stores them to wscale_out; otherwise
// they are read from wscale (the two pointers name the same buffer; a launch
// uses one of them).
template <int NW, bool FOLD>
__global__ void __launch_bounds__(kBlock)
    server_kernel(Part pt, int64_t L, int n, int64_t nseg, int64_t words,
                  const uint64_t* __restrict__ wbits, const float* __restrict__ wscale,
                  float* __restrict__ wscale_out, const double* __restrict__ wpart,
                  int64_t wcount, float* __restrict__ u, const float* __restrict__ sscale_prev,
                  uint64_t* __restrict__ sbits, double* __restrict__ spart) {
  const int lane = threadIdx.x & 63;
  const int j = pt.by0 + (int)blockIdx.y;
  // per-chunk worker scales: in registers for a compile-time count, staged
  // in LDS for a run-time one
  constexpr int WS = NW > 0 ? NW : 1;
  float ws[WS];
  __shared__ float sws[NW > 0 && !FOLD ? 1 : kMaxWorkersPerLaunch];
  if constexpr (FOLD) {
    fold_scales_in_block(wpart + (int64_t)j * wcount, (int64_t)n * wcount, wcount, n, L, sws,
                         wscale_out + j, n, pt.lo == 0 && pt.bx0 + blockIdx.x == 0);
  } else if constexpr (NW == 0) {
    if ((int)threadIdx.x < n) sws[threadIdx.x] = wscale[threadIdx.x * n + j];
    __syncthreads();
  }
  if constexpr (NW > 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w) ws[w] = FOLD ? uniform_f32(sws[w]) : wscale[w * n + j];
  }
  const float sp = sscale_prev[j];
  __shared__ double quad_part[kWavesPerBlock];
  const int64_t nquad = quads(nseg);
  {
    const int64_t qd = pt.bx0 + blockIdx.x;  // one quad per block
    const int64_t s = qd * kWavesPerBlock + wave_in_block();
    // one segment: its sum of squares after the butterfly
    auto segment = [&]() -> double {
      double acc = 0.0;
      const int64_t q0 = s * kSegElems;
      const int64_t left = (L - q0) >> 6;
      const int rows = left < kSegRows ? (int)left : kSegRows;
      const int64_t base = (int64_t)j * L + q0;
      const int64_t wbase = base >> 6;
      uint64_t mine = 0;
      if constexpr (NW > 0) {
        if (rows == kSegRows) {
          float up[kSegRows];
#pragma unroll
          for (int r = 0; r < kSegRows; ++r) up[r] = ld_stream(u + base + 64 * r + lane);
          float avg[kSegRows];
          server_average_segment<NW>(wbits, words, wbase, ws, avg);
#pragma unroll
          for (int r = 0; r < kSegRows; ++r) {
            const float e = up[r] - (up[r] >= 0.0f ? sp : -sp);
            const float uv = avg[r] + e;
            st_stream(u + base + 64 * r + lane, uv);
            const uint64_t word = __ballot(uv >= 0.0f);
            mine = lane == r ? word : mine;
            acc = add_square(acc, uv);
          }
          acc = butterfly(acc);
          if (lane < kSegRows) sbits[wbase + lane] = mine;
          return acc;
        }
      }
      for (int r = 0; r < rows; ++r) {
        const int64_t k = base + 64 * r + lane;
        const float up = u[k];
        const float e = up - (up >= 0.0f ? sp : -sp);
        const float a = worker_average<NW>(wbits, words, wbase + r, NW == 0 ? sws : ws, n);
        const float uv = a + e;
        u[k] = uv;
        const uint64_t word = __ballot(uv >= 0.0f);
        mine = lane == r ? word : mine;
        acc = add_square(acc, uv);
      }
      acc = butterfly(acc);
      if (lane < rows) sbits[wbase + lane] = mine;
      return acc;
    };
    store_quad_partial(s < nseg ? segment() : 0.0, quad_part, spart + (int64_t)j * nquad + qd);
  }
}

// ------------------------------------- server pass, 8 to 64 workers ----
// n = 8*NG workers.  Workers 4t..4t+3 form an aligned subtree of the
// pairwise tree, so their sum for one element depends only on their 4 sign
// bits: each block tabulates, in LDS, the 16 possible subtree sums of every
// such quad for its chunk's scales (each entry formed in the pairwise
// order), and the sum of an aligned 8-worker subtree is the sum of its two
// quads' entries -- the tree's next level.  A lookup's 64 lanes read one
// 16-entry table: 16 distinct words in 16 distinct banks, so no bank
// conflict (a table of all 256 sums of 8 workers was looked up at random
// words: its bank conflicts kept the LDS busy for 75 % of the n = 64 pass).
// The sign words are read with vector loads: for 8 rows, lane 8r + q loads
// worker 8g + q's word of row r, and a 64x64 bit transpose across the wave
// leaves in lane e, byte r, the 8 sign bits of workers 8g..8g+7 for element
// e of row r: two table indices.  The NG group sums are then added pairwise.
// (The scalar form needs one scalar load of 64 bytes per worker and 8 rows,
// and scalar loads do not overlap: with many workers it was bound by them.)

// One exchange stage of the transpose for one 32-bit half: bit K of the bit
// position swaps with bit K of the lane.  Lanes with bit K clear keep the
// positions with bit K clear and take the partner's (lane + K) others
// shifted up by K; lanes with bit K set keep the positions with bit K set and
// take the partner's (lane - K) others shifted down by K.  Every exchange is
// a VALU cross-lane operation (none goes through the LDS, which the table
// lookups keep busy):
//  - K = 16: gfx950's v_permlane16_swap of x with itself gives, in each lane,
//    x and its partner's x as the pair (lane with bit 4 clear: (own,
//    partner); set: (partner, own)); one byte permute with a per-lane
//    selector assembles the halfwords;
//  - K = 8: the partner's x by DPP row_ror:8 (lane ^ 8 within a 16-lane row),
//    one byte permute assembles the bytes;
//  - K = 4: the partner's x by DPP row_half_mirror then quad_perm [3,2,1,0]
//    (lane ^ 4), K = 2 and 1 by one quad_perm; rotations and a bit select
//    assemble the nibbles and bits (as rotations: the wrapped bits fall on
//    kept positions).
template <int K>
__device__ __forceinline__ uint32_t transpose_stage(uint32_t x, int lane) {
  const bool upper = (lane & K) != 0;
  if constexpr (K == 16) {
    const auto pr = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    // v_perm_b32(s0, s1, sel): selector bytes 0-3 take s1's bytes, 4-7 s0's
    return __builtin_amdgcn_perm(pr[1], pr[0], upper ? 0x07060302u : 0x05040100u);
  } else if constexpr (K == 8) {
    const uint32_t p = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);
    return __builtin_amdgcn_perm(p, x, upper ? 0x03070105u : 0x06020400u);
  } else {
    constexpr uint32_t kHigh = K == 4 ? 0xF0F0F0F0u : K == 2 ? 0xCCCCCCCCu : 0xAAAAAAAAu;
    uint32_t p;
    if constexpr (K == 4) {
      const int m = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
      p = (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);        // quad [3,2,1,0]
    } else if constexpr (K == 2) {
      p = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
    } else {
      p = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
    }
    const uint32_t r = __builtin_amdgcn_alignbit(p, p, upper ? K : 32 - K);
    const uint32_t keep = upper ? kHigh : ~kHigh;
    return (x & keep) | (r & ~keep);
  }
}

// 64x64 bit transpose across the wave.  On entry lane L holds row L of the
// matrix as (lo, hi) = bits 0..31 and 32..63; on exit lane e holds column e:
// bit L of (lo, hi) is bit e of row L.  (Every stage swaps one bit of the
// row index with the same bit of the column index; their order is free.)
__device__ __forceinline__ void transpose64(uint32_t& lo, uint32_t& hi, int lane) {
  // bit 5 of the position is the half: lanes 0..31 take the partner's (lane
  // + 32) lo as their hi, lanes 32..63 the partner's hi as their lo -- one
  // v_permlane32_swap (lo's upper 32 lanes trade with hi's lower 32)
  const auto sw = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
  lo = sw[0];
  hi = sw[1];
  lo = transpose_stage<16>(lo, lane);
  hi = transpose_stage<16>(hi, lane);
  lo = transpose_stage<8>(lo, lane);
  hi = transpose_stage<8>(hi, lane);
  lo = transpose_stage<4>(lo, lane);
  hi = transpose_stage<4>(hi, lane);
  lo = transpose_stage<2>(lo, lane);
  hi = transpose_stage<2>(hi, lane);
  lo = transpose_stage<1>(lo, lane);
  hi = transpose_stage<1>(hi, lane);
}

// Server average of rows 0..nrows-1 (nrows <= 8 used) starting at sign word
// `wrow0`, for lane's element: avg[r].  One worker's 16 words of a segment are
// one 128-byte line read in two halves, so these are ordinary loads (kept in
// L2 for the second half; non-temporal ones were 25 % slower).
template <int NG>
__device__ __forceinline__ void server_average_groups(const uint64_t* __restrict__ wbits,
                                                      int64_t words, int64_t wrow0, int nrows,
                                                      const float* tab, int lane, float* avg) {
  uint32_t lo[NG], hi[NG];
  const int q = lane & 7, r = lane >> 3;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    uint64_t wd = 0;
    if (r < nrows) wd = wbits[(int64_t)(8 * g + q) * words + wrow0 + r];
    lo[g] = (uint32_t)wd;
    hi[g] = (uint32_t)(wd >> 32);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) transpose64(lo[g], hi[g], lane);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    float o[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint32_t half = rr < 4 ? lo[g] : hi[g];
      o[g] = tab[32 * g + __builtin_amdgcn_ubfe(half, 8 * (rr & 3), 4)] +
             tab[32 * g + 16 + __builtin_amdgcn_ubfe(half, 8 * (rr & 3) + 4, 4)];
    }
    avg[rr] = pairwise_sum<NG>(o) / (float)(8 * NG);
  }
}

// The same average from a segment's sign words staged in LDS (see
// stage_segment_words): st holds, for workers 8k + a (k < NG, a < 8), the
// 16 words of the segment as 8 pieces of two rows, piece P of worker 8k + a
// at 16-byte slot 8k*8 + 8a + (P ^ a).  Lane 8r + q reads worker 8g + q's
// word of row 8h + r, one ds_read_b64: the xor spreads a read's 64 lanes
// evenly over the banks.
template <int NG>
__device__ __forceinline__ void server_average_groups_staged(const uint64_t* st, int h,
                                                             const float* tab, int lane,
                                                             float* avg) {
  uint32_t lo[NG], hi[NG];
  const int q = lane & 7, r = lane >> 3;
  const int slot = q * 16 + 2 * ((4 * h + (r >> 1)) ^ q) + (r & 1);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint64_t wd = st[g * 128 + slot];
    lo[g] = (uint32_t)wd;
    hi[g] = (uint32_t)(wd >> 32);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) transpose64(lo[g], hi[g], lane);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    float o[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint32_t half = rr < 4 ? lo[g] : hi[g];
      o[g] = tab[32 * g + __builtin_amdgcn_ubfe(half, 8 * (rr & 3), 4)] +
             tab[32 * g + 16 + __builtin_amdgcn_ubfe(half, 8 * (rr & 3) + 4, 4)];
    }
    avg[rr] = pairwise_sum<NG>(o) / (float)(8 * NG);
  }
}

// Copies the sign words of one segment (rows < 16 past a ragged chunk end)
// of all 8*NG workers into the wave's LDS area `st` with the gfx950 direct
// global-to-LDS load (16 bytes a lane, no registers): load k moves workers
// 8k..8k+7, lane 8a + b fetching piece b ^ a (rows 2(b^a), 2(b^a)+1) of
// worker 8k + a, so each worker's 128-byte line is read whole, once.  Pieces
// past a ragged end fetch the segment's first piece instead (in bounds; their
// rows are never used).  Needs 16-byte aligned words: an even number of rows
// per chunk.  Returns once the data is in LDS.
template <int NG>
__device__ __forceinline__ void stage_segment_words(const uint64_t* __restrict__ wbits,
                                                    int64_t words, int64_t wbase, int rows,
                                                    uint64_t* st, int lane) {
  const int a = lane >> 3, piece = (lane & 7) ^ a;
  const int64_t off = 2 * piece < rows ? 2 * piece : 0;
  // the wave's previous reads of st have returned before it is overwritten
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < NG; ++k)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(wbits + (int64_t)(8 * k + a) * words +
                                                        wbase + off),
        (__attribute__((address_space(3))) void*)(st + k * 128), 16, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// SEG_PARTIALS (32 and 64 workers, 4 segments per wave): a wave takes
// segments of the launch's range [pt.lo, pt.hi) strided by the launch's grid
// and stores one partial per segment.  Folding
// a quad's partials per block there needs a barrier per quad (the n = 64 pass
// went 6 % slower) or a wave-contiguous order (19 % more sign-word fetches).
// Otherwise the block's 4 waves take one segment each of a quad and fold
// their partials in LDS.
// FOLD as in server_kernel.  STAGE (chunks of an even number of rows): the
// sign words of each segment are staged in LDS whole (stage_segment_words)
// instead of being loaded half a line at a time.
template <int NG, bool SEG_PARTIALS, bool FOLD, bool STAGE>
__global__ void __launch_bounds__(kBlock)
    server_groups_kernel(Part pt, int64_t L, int n, int64_t nseg, int64_t words,
                         const uint64_t* __restrict__ wbits, const float* __restrict__ wscale,
                         float* __restrict__ wscale_out, const double* __restrict__ wpart,
                         int64_t wcount, float* __restrict__ u,
                         const float* __restrict__ sscale_prev, uint64_t* __restrict__ sbits,
                         double* __restrict__ spart) {
  __shared__ float tab[NG * 32];  // quad t of workers 4t..4t+3: tab[16t + its 4 sign bits]
  __shared__ uint64_t stage[STAGE ? kWavesPerBlock * NG * 128 : 1];
  // the folded worker scales are read only while the tables are built, before
  // the barrier that precedes any staging: with STAGE they share its area
  // (4 blocks of 40 KB fit a CU's 160 KB at 64 workers; 256 bytes more do not)
  __shared__ float sws_own[FOLD && !STAGE ? 8 * NG : 1];
  float* const sws = STAGE ? reinterpret_cast<float*>(stage) : sws_own;
  const int lane = threadIdx.x & 63;
  const int j = pt.by0 + (int)blockIdx.y;
  uint64_t* const st = stage + (STAGE ? wave_in_block() * NG * 128 : 0);
  if constexpr (FOLD)
    fold_scales_in_block(wpart + (int64_t)j * wcount, (int64_t)n * wcount, wcount, 8 * NG, L, sws,
                         wscale_out + j, n, pt.lo == 0 && pt.bx0 + blockIdx.x == 0);
  for (int t = threadIdx.x; t < NG * 32; t += kBlock) {
    const int qd = t >> 4, i = t & 15;
    float v[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float sc = FOLD ? sws[4 * qd + b] : wscale[(4 * qd + b) * n + j];
      v[b] = ((i >> b) & 1) ? sc : -sc;
    }
    tab[t] = pairwise_sum<4>(v);
  }
  __syncthreads();
  const float sp = sscale_prev[j];
  // one segment: its sum of squares after the butterfly
  auto segment = [&](int64_t s) -> double {
    const int64_t q0 = s * kSegElems;
    const int64_t left = (L - q0) >> 6;
    const int rows = left < kSegRows ? (int)left : kSegRows;
    const int64_t base = (int64_t)j * L + q0;
    const int64_t wbase = base >> 6;
    double acc = 0.0;
    uint64_t mine = 0;
    if constexpr (STAGE) stage_segment_words<NG>(wbits, words, wbase, rows, st, lane);
#pragma unroll
    for (int h = 0; h < kSegRows / 8; ++h) {
      const int nrows = rows - 8 * h;  // rows of this half (<= 0 past a chunk's end)
      if (nrows <= 0) break;
      float avg[8];
      if constexpr (STAGE)
        server_average_groups_staged<NG>(st, h, tab, lane, avg);
      else
        server_average_groups<NG>(wbits, words, wbase + 8 * h, nrows, tab, lane, avg);
      if (nrows >= 8) {
        float up[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) up[r] = ld_stream(u + base + 64 * (8 * h + r) + lane);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float e = up[r] - (up[r] >= 0.0f ? sp : -sp);
          const float uv = avg[r] + e;
          st_stream(u + base + 64 * (8 * h + r) + lane, uv);
          const uint64_t word = __ballot(uv >= 0.0f);
          mine = lane == 8 * h + r ? word : mine;
          acc = add_square(acc, uv);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r < nrows) {
            const int64_t k = base + 64 * (8 * h + r) + lane;
            const float up = u[k];
            const float e = up - (up >= 0.0f ? sp : -sp);
            const float uv = avg[r] + e;
            u[k] = uv;
            const uint64_t word = __ballot(uv >= 0.0f);
            mine = lane == 8 * h + r ? word : mine;
            acc = add_square(acc, uv);
          }
        }
      }
    }
    acc = butterfly(acc);
    if (lane < rows) sbits[wbase + lane] = mine;
    return acc;
  };
  if constexpr (SEG_PARTIALS) {
    const int64_t nwave = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t s = pt.lo + (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block(); s < pt.hi;
         s += nwave) {
      const double p = segment(s);
      if (lane == 0) spart[(int64_t)j * nseg + s] = p;
    }
  } else {
    __shared__ double quad_part[kWavesPerBlock];
    const int64_t nquad = quads(nseg);
    const int64_t qd = pt.bx0 + blockIdx.x;  // one quad per block
    const int64_t s = qd * kWavesPerBlock + wave_in_block();
    store_quad_partial(s < nseg ? segment(s) : 0.0, quad_part, spart + (int64_t)j * nquad + qd);
  }
}

// ------------------------------------------------------------------ update --
// m = (bit ? s_j : -s_j); x = x - lr * (m / (sqrtf(v) + eps)).  A wave owns 16
// consecutive rows of the flat vector; the chunk of a row is row*64 / L.
__device__ __forceinline__ float update_one(float x, float v, float mv, float lr, float eps) {
  return x - lr * (mv / (sqrtf(v) + eps));
}

// FOLD: the n server scales are folded by every block from the server pass's
// partials (`scount` per row) and the grid's first block stores them to
// sscale_out; otherwise they are read from sscale (the same buffer).
template <bool FOLD>
__global__ void __launch_bounds__(kBlock)
    update_kernel(Part pt, int64_t words, int64_t L, int n, const uint64_t* __restrict__ sbits,
                  const float* __restrict__ sscale, float* __restrict__ sscale_out,
                  const double* __restrict__ spart, int64_t scount, const float* __restrict__ v,
                  float* __restrict__ x, float lr, float eps) {
  const int lane = threadIdx.x & 63;
  __shared__ float fss[FOLD ? kMaxWorkersPerLaunch : 1];
  if constexpr (FOLD)
    fold_scales_in_block(spart, scount, scount, n, L, fss, sscale_out, 1,
                         pt.lo == 0 && blockIdx.x == 0);
  auto scale_of = [&](int64_t jj) -> float {
    if constexpr (FOLD) return fss[jj];
    return sscale[jj];
  };
  const int64_t nwave = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t rows_per_chunk = L >> 6;
  for (int64_t gi = pt.lo + (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block(); gi < pt.hi;
       gi += nwave) {
    const int64_t r0 = gi * kSegRows;
    const int rows = words - r0 < kSegRows ? (int)(words - r0) : kSegRows;
    const int64_t j0 = r0 / rows_per_chunk;
    // the 16 rows lie in one chunk unless a chunk boundary falls inside them
    const bool one_chunk = rows == kSegRows && (r0 + kSegRows - 1) / rows_per_chunk == j0;
    if (one_chunk) {
      const float s = scale_of(j0);
      float xv[kSegRows], vv[kSegRows];
#pragma unroll
      for (int r = 0; r < kSegRows; ++r) {
        xv[r] = ld_stream(x + (r0 + r) * 64 + lane);
        vv[r] = ld_stream(v + (r0 + r) * 64 + lane);
      }
#pragma unroll
      for (int r = 0; r < kSegRows; ++r)
        st_stream(x + (r0 + r) * 64 + lane,
                  update_one(xv[r], vv[r], signed_scale(sbits[r0 + r], s), lr, eps));
    } else {
      for (int r = 0; r < rows; ++r) {
        const int64_t row = r0 + r;
        const float s = scale_of(row / rows_per_chunk);
        const int64_t k = row * 64 + lane;
        x[k] = update_one(x[k], v[k], signed_scale(sbits[row], s), lr, eps);
      }
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

// A worker's local model inside an open 0/1 period: x_sync - G*(a/(sqrtf(v)+eps)).
__global__ void __launch_bounds__(kBlock)
    zo_local_model_kernel(const float* __restrict__ x, const float* __restrict__ a,
                          const float* __restrict__ v, float gamma, float eps, int64_t offset,
                          int64_t count, float* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count; i += stride) {
    const int64_t k = offset + i;
    dst[i] = x[k] - gamma * (a[k] / (sqrtf(v[k]) + eps));
  }
}

// Every launch goes through the runtime's extended launch so that timing
// events, when requested, are taken from the dispatch packet itself (no extra
// packets between kernels); with null events it is a plain launch.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  hipEvent_t t0, hipEvent_t t1, Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t0, t1, 0, args...);
  return hipGetLastError();
}

unsigned grid_for(int64_t items, int64_t per_block, int64_t cap) {
  int64_t b = (items + per_block - 1) / per_block;
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return (unsigned)b;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Elements of a streaming pass per launch.  On MI355X a pass moves more
// bytes per second as a sequence of launches of tens of millions of
// elements than as one launch over billions: a 2^31-element fp32
// read-modify-write probe ran at 5.8 TB/s as one launch, 6.1 TB/s as 8
// launches and 6.4 TB/s as 64 launches of 2^25 (512 launches of 2^22 fell to
// 5.4 TB/s on their gaps).  On the step itself (sizes 2^24 to 2^27 and
// unsplit, measured on 110M x 8 bf16, 334M x 16, 1.56G x 8 and 340M x 64)
// launches of 2^26 and 2^27 were best: 4-5 % off the step where one launch
// covered 5-12 G elements, neutral where launches were already 340M.  The
// server pass for 32 and 64 workers, whose waves take 4 segments each, lost
// to tails when cut (1.05 -> 1.17 ms on 340M x 64 at 2^26): it is cut only
// past kSegPartialLaunchScale times the size.
constexpr int64_t kLaunchElems = int64_t(1) << 26;
constexpr int64_t kSegPartialLaunchScale = 16;
// s.launch_elems (a debug setting) applies to every pass unscaled.
int64_t per_launch(const State& s, int64_t scale = 1) {
  return s.launch_elems > 0 ? s.launch_elems : kLaunchElems * scale;
}

// Issues a pass over `rows` grid rows of `nbx` blocks, each row `row_elems`
// elements, as launches of about per_launch(s) elements: whole rows grouped,
// or, for rows of more than that, ranges of a row's blocks.  one(part, grid,
// t0, t1) makes one launch; the pass's start event goes with its first
// launch and its end event with its last, so they time the whole pass.
template <typename F>
hipError_t launch_parts(const State& s, int rows, int64_t nbx, int64_t row_elems, hipEvent_t t0,
                        hipEvent_t t1, F one, int64_t scale = 1) {
  const int64_t elems = per_launch(s, scale);
  const int64_t total = (int64_t)rows * row_elems;
  int64_t cuts = 1;      // parts of one row
  int per_rows = rows;   // rows of one part
  if (total > elems) {
    if (row_elems >= elems) {
      cuts = std::min<int64_t>(nbx, (row_elems + elems - 1) / elems);
      per_rows = 1;
    } else {
      const int64_t parts = (total + elems - 1) / elems;
      per_rows = (int)((rows + parts - 1) / parts);
    }
  }
  const int64_t bx_per = (nbx + cuts - 1) / cuts;
  for (int r0 = 0; r0 < rows; r0 += per_rows) {
    const int nr = std::min(per_rows, rows - r0);
    for (int64_t b0 = 0; b0 < nbx; b0 += bx_per) {
      const int64_t nb = std::min(bx_per, nbx - b0);
      const bool first = r0 == 0 && b0 == 0;
      const bool last = r0 + nr == rows && b0 + nb == nbx;
      const hipError_t e = one(Part{b0, r0, 0, 0}, dim3((unsigned)nb, (unsigned)nr),
                               first ? t0 : nullptr, last ? t1 : nullptr);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// The same for a pass whose waves stride over `items` work items of
// `item_elems` elements each, `per_wave` items a wave: ranges [lo, hi) of
// about per_launch(s) elements, each launched with enough blocks to give
// every wave per_wave items (at most `cap` blocks).
template <typename F>
hipError_t launch_ranges(const State& s, int64_t items, int64_t item_elems, int per_wave,
                         int64_t cap, hipEvent_t t0, hipEvent_t t1, F one) {
  const int64_t elems = per_launch(s);
  const int64_t total = items * item_elems;
  const int64_t parts = std::max<int64_t>(1, (total + elems - 1) / elems);
  const int64_t per = std::max<int64_t>(1, (items + parts - 1) / parts);
  for (int64_t lo = 0;; lo += per) {
    const int64_t hi = std::min(items, lo + per);
    const dim3 grid(grid_for(hi - lo, kWavesPerBlock * per_wave, cap));
    const hipError_t e = one(Part{0, 0, lo, hi}, grid, lo == 0 ? t0 : nullptr,
                             hi == items ? t1 : nullptr);
    if (e != hipSuccess || hi == items) return e;
  }
}

}  // namespace

Layout layout_for(int64_t d, int n, bool zero_one) {
  Layout l{};
  const uint64_t ud = (uint64_t)d, un = (uint64_t)n;
  const uint64_t nseg = (uint64_t)((d / n + kSegElems - 1) / kSegElems);
  uint64_t off = 0;
  int ng = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    l.guard[ng++] = at + bytes;  // right after the buffer (4-byte aligned)
    off = align256(at + bytes + kGuardBytes);
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
  l.fold = take(8 * un * un * (uint64_t)fold_doubles_per_row((int64_t)nseg));
  l.wscale = take(4 * un * un);
  l.sscale = take(4 * un);
  l.mloc = take(zero_one ? 4 * ud * un : 0);
  l.aloc = take(zero_one ? 4 * ud * un : 0);
  l.total = off;
  return l;
}

ScratchLayout scratch_layout(int64_t nseg, int n) {
  const uint64_t un = (uint64_t)n;
  const int64_t wrow = quads(nseg);  // worker rows: one partial per block of 4 segments
  const int64_t srow = server_segment_partials(n) ? nseg : quads(nseg);
  const uint64_t wfold = un * un * (uint64_t)fold_doubles_per_row(wrow);
  const uint64_t sfold = un * (uint64_t)fold_doubles_per_row(srow);
  ScratchLayout l{};
  l.wpart = 0;
  l.spart = align256(l.wpart + 8 * un * un * (uint64_t)wrow);
  l.fold = align256(l.spart + 8 * un * (uint64_t)srow);
  l.total = align256(l.fold + 8 * (wfold > sfold ? wfold : sfold));
  return l;
}

hipError_t launch_warmup(const State& s, const GradPtrs& g, float lr, float bc1, float bc2,
                         hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const float ob1 = 1.0f - s.beta1, ob2 = 1.0f - s.beta2;
  const dim3 grid(grid_for(s.d, kBlock, 8192));
  // one wave per group of rows: ceil(words / R) waves, R from the worker count
  const int64_t R = s.n <= 8 ? 4 : (s.n <= 16 ? 2 : 1);
  const dim3 rows_grid(grid_for((s.words + R - 1) / R, kWavesPerBlock, kMaxBlocksPerRow));
#define OB_WARM(GT, NW)                                                                         \
  if (NW > 0)                                                                                   \
    return launch(warmup_rows_kernel<GT, (NW > 0 ? NW : 1)>, rows_grid, dim3(kBlock), stream,   \
                  t0, t1, g, s.words, s.m, s.v, s.x, s.beta1, ob1, s.beta2, ob2, bc1, bc2, lr,  \
                  s.eps);                                                                       \
  return launch(warmup_kernel<GT, NW>, grid, dim3(kBlock), stream, t0, t1, g, s.n, s.d, s.m,     \
                s.v, s.x, s.beta1, ob1, s.beta2, ob2, bc1, bc2, lr, s.eps)
#define OB_WARM_N(GT)                \
  switch (s.n) {                     \
    case 1: OB_WARM(GT, 1);          \
    case 2: OB_WARM(GT, 2);          \
    case 4: OB_WARM(GT, 4);          \
    case 8: OB_WARM(GT, 8);          \
    case 16: OB_WARM(GT, 16);        \
    case 32: OB_WARM(GT, 32);        \
    case 64: OB_WARM(GT, 64);        \
    default: OB_WARM(GT, 0);         \
  }
  if (s.grad_bf16) {
    OB_WARM_N(uint16_t)
  } else {
    OB_WARM_N(float)
  }
#undef OB_WARM_N
#undef OB_WARM
}

int warmup_stack_levels(int n) {
  int levels = 0;
  while ((1 << levels) <= n) ++levels;  // floor(log2(n)) + 1
  return levels;
}

hipError_t launch_warmup_push(const State& s, const void* grad, int worker, hipStream_t stream,
                              hipEvent_t t0, hipEvent_t t1) {
  int merges = 0;
  while ((worker >> merges) & 1) ++merges;
  const dim3 grid(grid_for(s.d, kBlock, 8192));
  if (s.grad_bf16)
    return launch(warmup_push_kernel<uint16_t>, grid, dim3(kBlock), stream, t0, t1,
                  (const uint16_t*)grad, s.c, s.d, merges);
  return launch(warmup_push_kernel<float>, grid, dim3(kBlock), stream, t0, t1,
                (const float*)grad, s.c, s.d, merges);
}

hipError_t launch_warmup_finish(const State& s, float lr, float bc1, float bc2,
                                hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const float ob1 = 1.0f - s.beta1, ob2 = 1.0f - s.beta2;
  return launch(warmup_finish_kernel, dim3(grid_for(s.d, kBlock, 8192)), dim3(kBlock), stream, t0,
                t1, s.c, s.d, s.n, warmup_stack_levels(s.n), s.m, s.v, s.x, s.beta1, ob1,
                s.beta2, ob2, bc1, bc2, lr, s.eps);
}

// Workers per block of the first-step kernels: all nw of the launch, sharing
// each segment of m, where the chunks hold enough quads for several rounds
// of blocks without splitting by worker; else one (on 1M parameters x 4
// workers, 256 blocks of 4 workers took 20 us against 12 us for 1024 blocks
// of one).
constexpr int64_t kShareMinBlocks = 4096;
int first_group(const State& s, int nw) {
  return (int64_t)s.n * quads(s.nseg) >= kShareMinBlocks ? nw : 1;
}

hipError_t launch_worker_pass(const State& s, const GradPtrs& g, int w0, int nw, bool m_bits,
                              hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const float ob1 = 1.0f - s.beta1;
  if (!m_bits) {
    // grid rows: (worker group, chunk).  Launches are sized by elements of m
    // (a wave's loop over its group is serial, so a launch needs several
    // rounds of waves to keep the memory busy)
    const int wg = first_group(s, nw);
    auto kernel = s.grad_bf16 ? worker_first_kernel<uint16_t> : worker_first_kernel<float>;
    return launch_parts(s, nw / wg * s.n, quads(s.nseg), s.L, t0, t1,
                        [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                          return launch(kernel, grid, dim3(kBlock), stream, a, b, g, w0, wg, pt,
                                        s.d, s.L, s.n, s.nseg, s.words, (const float*)s.m, s.c,
                                        (const float*)s.wscale, s.wbits, s.wpart, s.beta1, ob1);
                        });
  }
  auto kernel = s.grad_bf16 ? worker_kernel<uint16_t> : worker_kernel<float>;
  // grid rows: (worker, chunk), one block per quad of the chunk's segments
  return launch_parts(s, nw * s.n, quads(s.nseg), s.L, t0, t1,
                      [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                        return launch(kernel, grid, dim3(kBlock), stream, a, b, g, w0, pt, s.d,
                                      s.L, s.n, s.nseg, s.words, (const uint64_t*)s.sbits,
                                      (const float*)s.sscale, s.c, (const float*)s.wscale,
                                      s.wbits, s.wpart, s.beta1, ob1);
                      });
}

hipError_t launch_zo_local(const State& s, const GradPtrs& g, bool first, bool m_bits, float wk,
                           hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const float ob1 = 1.0f - s.beta1;
  if (first && !m_bits) {
    // grid rows: (worker group, chunk); launches sized by elements of m, as
    // for worker_first_kernel
    const int wg = first_group(s, s.n);
    auto kernel = s.grad_bf16 ? zo_local_first_kernel<uint16_t> : zo_local_first_kernel<float>;
    return launch_parts(s, s.n / wg * s.n, quads(s.nseg), s.L, t0, t1,
                        [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                          return launch(kernel, grid, dim3(kBlock), stream, a, b, g, wg, pt, s.d,
                                        s.L, s.n, s.nseg, (const float*)s.m, s.mloc, s.aloc,
                                        s.beta1, ob1);
                        });
  }
  // FIRST and MBITS: the shared momentum is read only at a period's first
  // step, and is held as server sign words after the first synchronization
  auto kernel = s.grad_bf16 ? (first ? zo_local_kernel<uint16_t, true, true>
                                     : zo_local_kernel<uint16_t, false, false>)
                            : (first ? zo_local_kernel<float, true, true>
                                     : zo_local_kernel<float, false, false>);
  return launch_parts(s, s.n * s.n, quads(s.nseg), s.L, t0, t1,
                      [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                        return launch(kernel, grid, dim3(kBlock), stream, a, b, g, pt, s.d, s.L,
                                      s.n, s.nseg, (const float*)s.m, (const uint64_t*)s.sbits,
                                      (const float*)s.sscale, s.mloc, s.aloc, s.beta1, ob1, wk);
                      });
}

hipError_t launch_zo_sync(const State& s, const GradPtrs& g, bool first, bool m_bits, float wk,
                          hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const float ob1 = 1.0f - s.beta1;
  auto kernel =
      s.grad_bf16
          ? (!first ? zo_sync_kernel<uint16_t, false, false>
                    : m_bits ? zo_sync_kernel<uint16_t, true, true>
                             : zo_sync_kernel<uint16_t, true, false>)
          : (!first ? zo_sync_kernel<float, false, false>
                    : m_bits ? zo_sync_kernel<float, true, true> : zo_sync_kernel<float, true, false>);
  return launch_parts(s, s.n * s.n, quads(s.nseg), s.L, t0, t1,
                      [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                        return launch(kernel, grid, dim3(kBlock), stream, a, b, g, pt, s.d, s.L,
                                      s.n, s.nseg, s.words, (const float*)s.m,
                                      (const uint64_t*)s.sbits, (const float*)s.sscale,
                                      (const float*)s.mloc, (const float*)s.aloc, s.c,
                                      (const float*)s.wscale, s.wbits, s.wpart, s.beta1, ob1, wk);
                      });
}

hipError_t launch_zo_refresh(const State& s, const GradPtrs& g, hipStream_t stream,
                             hipEvent_t t0, hipEvent_t t1) {
  const float ob2 = 1.0f - s.beta2;
  const dim3 grid(grid_for(s.d, kBlock, 8192));
#define OB_ZOR(GT, NW)                                                                         \
  return launch(zo_refresh_kernel<GT, NW>, grid, dim3(kBlock), stream, t0, t1, g, s.n, s.d, s.v, \
                s.beta2, ob2)
#define OB_ZOR_N(GT)          \
  switch (s.n) {              \
    case 1: OB_ZOR(GT, 1);    \
    case 2: OB_ZOR(GT, 2);    \
    case 4: OB_ZOR(GT, 4);    \
    case 8: OB_ZOR(GT, 8);    \
    case 16: OB_ZOR(GT, 16);  \
    default: OB_ZOR(GT, 0);   \
  }
  if (s.grad_bf16) {
    OB_ZOR_N(uint16_t)
  } else {
    OB_ZOR_N(float)
  }
#undef OB_ZOR_N
#undef OB_ZOR
}

// Scales of `rows` rows of partials (`nseg` per row: one per segment, or one
// per block of 4 segments, whose pairwise sums continue the same tree) into
// scale_out: fold aligned groups of kGroup until at most kGroup values remain
// per row, then the last fold and the scale.  `fold` holds rows *
// fold_doubles_per_row(nseg) doubles.  t0 is taken at the first launch, t1
// at the last.
static hipError_t launch_scales(const double* part, int64_t nseg, int64_t L, int rows,
                                double* fold, float* scale_out, hipStream_t stream,
                                hipEvent_t t0, hipEvent_t t1) {
  int64_t width = 1;
  while (width < nseg) width <<= 1;
  // one dispatch for moderate rows; with thousands of rows (n*n worker rows at
  // large n) the parallel group fold below keeps more waves busy
  if (width > kGroup && width <= (int64_t)kBlock * 64 && rows <= 512) {
    const dim3 grid((unsigned)rows), block(kBlock);
    if (width <= (int64_t)kBlock * 4)
      return launch(scale_direct_kernel<4>, grid, block, stream, t0, t1, part, nseg, L, scale_out);
    if (width <= (int64_t)kBlock * 8)
      return launch(scale_direct_kernel<8>, grid, block, stream, t0, t1, part, nseg, L, scale_out);
    if (width <= (int64_t)kBlock * 16)
      return launch(scale_direct_kernel<16>, grid, block, stream, t0, t1, part, nseg, L,
                    scale_out);
    if (width <= (int64_t)kBlock * 32)
      return launch(scale_direct_kernel<32>, grid, block, stream, t0, t1, part, nseg, L,
                    scale_out);
    return launch(scale_direct_kernel<64>, grid, block, stream, t0, t1, part, nseg, L, scale_out);
  }
  // a row of at most kGroup partials: one block per row
  if (width <= kGroup)
    return launch(scale_kernel, dim3((unsigned)rows), dim3(kBlock), stream, t0, t1, part, nseg, L,
                  scale_out);
  // longer rows: aligned groups of kGroup partials folded in parallel, then
  // one block per row folds the group results (at most kGroup of them: a
  // row holds at most kGroup^2 partials, by the shape rule)
  const int64_t ngroups = width / kGroup;
  hipError_t e = launch(fold_groups_kernel, dim3((unsigned)ngroups, (unsigned)rows), dim3(kBlock),
                        stream, t0, nullptr, part, nseg, ngroups, fold);
  if (e != hipSuccess) return e;
  return launch(scale_kernel, dim3((unsigned)rows), dim3(kBlock), stream, nullptr, t1,
                (const double*)fold, ngroups, L, scale_out);
}

// Partials per row left by the worker pass (one per block of 4 segments) and
// by the server pass (the same, or one per segment with 32 and 64 workers).
static int64_t worker_row_partials(const State& s) { return quads(s.nseg); }
static int64_t server_row_partials(const State& s) {
  return server_segment_partials(s.n) ? s.nseg : quads(s.nseg);
}

bool scales_in_consumers(const State& s) {
  const int64_t longest = std::max(worker_row_partials(s), server_row_partials(s));
  return longest <= 64 && (int64_t)s.n * longest <= 1024;
}

hipError_t launch_worker_scales(const State& s, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  return launch_scales(s.wpart, worker_row_partials(s), s.L, s.n * s.n, s.fold, s.wscale, stream,
                       t0, t1);
}

using ServerKernel = void (*)(Part, int64_t, int, int64_t, int64_t, const uint64_t*,
                              const float*, float*, const double*, int64_t, float*, const float*,
                              uint64_t*, double*);

template <int NG, bool WQ>
ServerKernel server_groups_for(bool fold, bool stage) {
  if (fold)
    return stage ? server_groups_kernel<NG, WQ, true, true> : server_groups_kernel<NG, WQ, true, false>;
  return stage ? server_groups_kernel<NG, WQ, false, true> : server_groups_kernel<NG, WQ, false, false>;
}

template <int NW>
ServerKernel server_for(bool fold) {
  return fold ? server_kernel<NW, true> : server_kernel<NW, false>;
}

hipError_t launch_server_pass(const State& s, bool fold_scales, bool stage_words,
                              hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const int64_t wcount = worker_row_partials(s);
  auto run = [&](ServerKernel k, Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
    return launch(k, grid, dim3(kBlock), stream, a, b, pt, s.L, s.n, s.nseg, s.words,
                  (const uint64_t*)s.wbits, (const float*)s.wscale, s.wscale,
                  (const double*)s.wpart, wcount, s.u, (const float*)s.sscale, s.sbits, s.spart);
  };
  if (s.n == 8 || s.n == 16 || s.n == 32 || s.n == 64) {
    // staging in LDS needs 16-byte aligned sign words: an even number of
    // rows per chunk
    const bool stage = stage_words && ((s.L >> 6) & 1) == 0;
    const ServerKernel k = s.n == 8    ? server_groups_for<1, false>(fold_scales, stage)
                           : s.n == 16 ? server_groups_for<2, false>(fold_scales, stage)
                           : s.n == 32 ? server_groups_for<4, server_segment_partials(32)>(
                                             fold_scales, stage)
                                       : server_groups_for<8, server_segment_partials(64)>(
                                             fold_scales, stage);
    if (!server_segment_partials(s.n))  // one quad per block, as the worker pass
      return launch_parts(s, s.n, quads(s.nseg), s.L, t0, t1,
                          [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                            return run(k, pt, grid, a, b);
                          });
    // 32 and 64 workers: waves take 4 segments each of the part's segment
    // range [lo, hi), strided by the launch (the tables are built once per
    // block)
    return launch_parts(s, s.n, s.nseg, s.L, t0, t1,
                        [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                          const Part seg{0, pt.by0, pt.bx0, pt.bx0 + (int64_t)grid.x};
                          const dim3 g(grid_for(grid.x, kWavesPerBlock * 4, kMaxBlocksPerRow),
                                       grid.y);
                          return run(k, seg, g, a, b);
                        },
                        kSegPartialLaunchScale);
  }
  const ServerKernel k = s.n == 1   ? server_for<1>(fold_scales)
                         : s.n == 2 ? server_for<2>(fold_scales)
                         : s.n == 4 ? server_for<4>(fold_scales)
                                    : server_for<0>(fold_scales);
  return launch_parts(s, s.n, quads(s.nseg), s.L, t0, t1,
                      [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                        return run(k, pt, grid, a, b);
                      });
}

hipError_t launch_server_scales(const State& s, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  return launch_scales(s.spart, server_row_partials(s), s.L, s.n, s.fold, s.sscale, stream, t0,
                       t1);
}

hipError_t launch_update(const State& s, float lr, bool fold_scales, hipStream_t stream,
                         hipEvent_t t0, hipEvent_t t1) {
  const int64_t groups = (s.words + kSegRows - 1) / kSegRows;  // of 16 rows, one wave each
  auto kernel = fold_scales ? update_kernel<true> : update_kernel<false>;
  return launch_ranges(s, groups, kSegElems, 1, kMaxBlocksPerRow, t0, t1,
                       [&](Part pt, dim3 grid, hipEvent_t a, hipEvent_t b) {
                         return launch(kernel, grid, dim3(kBlock), stream, a, b, pt, s.words,
                                       s.L, s.n, (const uint64_t*)s.sbits,
                                       (const float*)s.sscale, s.sscale,
                                       (const double*)s.spart, server_row_partials(s),
                                       (const float*)s.v, s.x, lr, s.eps);
                       });
}

hipError_t launch_error_out(const float* comp, const float* scales, int64_t L, int64_t offset,
                            int64_t count, float* dst, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  return launch(error_out_kernel, dim3(grid_for(count, kBlock, 16384)), dim3(kBlock), stream,
                nullptr, nullptr, comp, scales, L, offset, count, dst);
}

hipError_t launch_zo_local_model(const float* x, const float* a, const float* v, float gamma,
                                float eps, int64_t offset, int64_t count, float* dst,
                                hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  return launch(zo_local_model_kernel, dim3(grid_for(count, kBlock, 16384)), dim3(kBlock), stream,
                nullptr, nullptr, x, a, v, gamma, eps, offset, count, dst);
}

hipError_t launch_decompress_out(const uint64_t* bits, const float* scales, int64_t L,
                                 int64_t offset, int64_t count, float* dst, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  return launch(decompress_out_kernel, dim3(grid_for(count, kBlock, 16384)), dim3(kBlock), stream,
                nullptr, nullptr, bits, scales, L, offset, count, dst);
}

}  // namespace ob
