// Launchers of the gfx950 kernels behind the ob_adam C interface.
// Internal to the library; every launcher enqueues on `stream` and returns
// hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ob {

constexpr int kMaxWorkersPerLaunch = 64;
constexpr int kSegElems = 1024;   // elements of one fixed-order segment (one wavefront)
constexpr int kSegRows = 16;      // rows of 64 elements per segment
constexpr int64_t kMaxSegsPerChunk = int64_t(1) << 20;  // chunks of at most 2^30 elements
// With 32 and 64 workers the server pass leaves one partial per segment, and
// its finalize folds at most 2^18 of them: chunks of at most 2^28 elements.
constexpr int64_t kMaxSegsPerChunkSegPartials = int64_t(1) << 18;

struct GradPtrs {
  const void* p[kMaxWorkersPerLaunch];
};

// Device state carved out of the caller's workspace.
struct State {
  int64_t d, L, nseg, words;  // words = d/64
  int n;
  int64_t launch_elems;  // elements per launch of a streaming pass (0: the default)
  int grad_bf16;
  float beta1, beta2, eps;
  float* x;
  float* m;
  float* v;
  float* u;           // [d]     server: last compensated average (error is derived)
  float* c;           // [n][d]  worker: last compensated momentum (error is derived)
  uint64_t* wbits;    // [n][words]
  uint64_t* sbits;    // [words]
  double* wpart;      // [n][n][nseg] segment partials of the worker sums of squares
  double* spart;      // [n][nseg]
  double* fold;       // [n][n][groups] group results of the scale finalize
  float* wscale;      // [n][n] row i = worker i, column j = chunk j
  float* sscale;      // [n]
  float* mloc;        // [n][d]  0/1 Adam: each worker's local momentum (else null)
  float* aloc;        // [n][d]  0/1 Adam: each worker's step-weighted mean momentum
};

// Workspace layout: byte offsets of each buffer (256-byte aligned) and total.
// Every sub-buffer is followed directly by a guard region of kGuardBytes
// holding a known pattern (guard i: 32-bit words guard_word(i)), so that a
// write past a buffer's end can be detected from the host.
constexpr int kNumGuards = 14;
constexpr uint64_t kGuardBytes = 256;
constexpr uint32_t guard_word(int i) { return 0xA5C30000u + (uint32_t)i; }

struct Layout {
  uint64_t x, m, v, u, c, wbits, sbits, wpart, spart, fold, wscale, sscale, mloc, aloc, total;
  uint64_t guard[kNumGuards];  // offsets of the guards, in workspace order
};
// zero_one: the 0/1 Adam variant's two per-worker slabs are reserved (else
// they take no bytes; their guards are still there).
Layout layout_for(int64_t d, int n, bool zero_one);

// The step's scratch (fixed-order partials of the workers and the server and
// the finalize's group results) laid out in one region of its own: byte
// offsets (256-byte aligned) and total.  layout_for reserves the same
// buffers (at least as large) inside the workspace.
struct ScratchLayout {
  uint64_t wpart, spart, fold, total;
};
ScratchLayout scratch_layout(int64_t nseg, int n);

// t0 / t1: optional timing events recorded at the start of the first and the
// end of the last dispatch of the launcher (null = untimed).
hipError_t launch_warmup(const State& s, const GradPtrs& g, float lr, float bc1, float bc2,
                         hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
// Worker-at-a-time warm-up: the binary-counter stack of partial gradient sums
// lives in the compensated slabs (levels 0..warmup_stack_levels(n)-1 of d
// floats each, at most n), which the finish clears again.
int warmup_stack_levels(int n);
hipError_t launch_warmup_push(const State& s, const void* grad, int worker, hipStream_t stream,
                              hipEvent_t t0, hipEvent_t t1);
hipError_t launch_warmup_finish(const State& s, float lr, float bc1, float bc2,
                                hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_worker_pass(const State& s, const GradPtrs& g, int w0, int nw, bool m_bits,
                              hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
// Whether a step's per-chunk scales can be folded by the passes that consume
// them -- every server block its chunk's worker rows, every update block the
// server rows -- instead of by dispatches of their own: rows of at most 64
// partials, and at most 1024 partials read per block.  The scales are the
// same bits either way.  With fold_scales, launch_server_pass and
// launch_update do it and launch_worker_scales / launch_server_scales are not
// called.
bool scales_in_consumers(const State& s);
hipError_t launch_worker_scales(const State& s, hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
// stage_words: the 8-64-worker form stages each segment's sign words in LDS
// (chunks of an even number of rows; others, or false, load them directly).
// The same bits either way.
hipError_t launch_server_pass(const State& s, bool fold_scales, bool stage_words,
                              hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_server_scales(const State& s, hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_update(const State& s, float lr, bool fold_scales, hipStream_t stream,
                         hipEvent_t t0, hipEvent_t t1);
// 0/1 Adam: a local step of all workers (first: the first step of a local
// period; m_bits: the shared momentum is held as server sign words), the
// synchronizing step's worker pass (then worker scales, server pass, server
// scales and launch_update with the period's summed step sizes), and the
// variance refresh.  wk = lr / (the period's summed step sizes so far).
hipError_t launch_zo_local(const State& s, const GradPtrs& g, bool first, bool m_bits, float wk,
                           hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_zo_sync(const State& s, const GradPtrs& g, bool first, bool m_bits, float wk,
                          hipStream_t stream, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_zo_refresh(const State& s, const GradPtrs& g, hipStream_t stream,
                             hipEvent_t t0, hipEvent_t t1);

// Materialize derived fields for readback.
hipError_t launch_error_out(const float* comp, const float* scales, int64_t L, int64_t offset,
                            int64_t count, float* dst, hipStream_t stream);
hipError_t launch_decompress_out(const uint64_t* bits, const float* scales, int64_t L,
                                 int64_t offset, int64_t count, float* dst, hipStream_t stream);
hipError_t launch_zo_local_model(const float* x, const float* a, const float* v, float gamma,
                                float eps, int64_t offset, int64_t count, float* dst,
                                hipStream_t stream);

}  // namespace ob
