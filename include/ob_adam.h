/*
 * ob_adam: the compression-phase step of 1-bit Adam on one MI355X (gfx950).
 *
 * Method: "1-bit Adam: Communication Efficient Large-Scale Training with
 * Adam's Convergence Speed" (Abstract): full-precision Adam for a warm-up,
 * then a compression phase in which Adam's variance is a fixed
 * preconditioner and the momentum is sent with error-compensated 1-bit
 * compression.  "LIT-278: 1-bit Adam ..." (Key takeaways, Theorem 1
 * conditions): per-chunk scaling; tag lines SOTA-214 (error feedback on the
 * momentum) and SOTA-215 (freeze the variance, compress the momentum and
 * never the update); "What the evidence does not cover" (the compressed
 * allreduce).
 *
 * n data-parallel workers are simulated as n state slabs in one GPU's HBM;
 * the compressed allreduce is its arithmetic only (worker compress, server
 * chunk-average and re-compress with server error feedback, decompress).
 *
 * Arithmetic contract (the same for every entry point):
 *  - d parameters, n workers, chunk length L = d/n; chunk j = [j*L, (j+1)*L)
 *    is server j's share and the unit of every worker's scaling.
 *  - warm-up step t (1-based): gbar = pairwise-by-levels sum of the n
 *    gradients (pairs (2i,2i+1), an odd tail passes up) / (float)n;
 *    m = (b1*m) + ((1-b1)*gbar); v = (b2*v) + ((1-b2)*(gbar*gbar));
 *    x = x - lr*((m/bc1) / (sqrtf(v/bc2) + eps)), bc = (float)(1 - b^t) with
 *    b^t formed by t fp64 multiplications.
 *  - compressed step: per worker i and element, c = ((b1*m) + ((1-b1)*g_i))
 *    + e_i; per (i, chunk j) scale s_ij = (float)(sqrt(S)/sqrt((double)L)),
 *    S = fp64 sum of c^2 in the fixed order described below; sign bit =
 *    (c >= 0); e_i = c - (bit ? s_ij : -s_ij).  Server j: a = pairwise sum
 *    over workers of (bit ? s_ij : -s_ij) / (float)n; u = a + e_srv; scale
 *    s_j from u the same way; e_srv = u - (u >= 0 ? s_j : -s_j); m = (u >= 0
 *    ? s_j : -s_j); x = x - lr*(m / (sqrtf(v) + eps)); v unchanged.
 *  - fixed fp64 order of a chunk's sum of squares: segments of 1024
 *    elements; accumulator k of a segment adds the squares of elements
 *    1024*s + 64*r + k for r = 0..15 in turn; then an xor butterfly over the
 *    64 accumulators with offsets 32,16,8,4,2,1; then a pairwise sum over the
 *    segment partials padded with zeros to a power of two.
 *  - sign words: element k of a d-vector is bit k%64 of uint64 word k/64.
 *  - no fused multiply-add contraction, no flush of denormals, correctly
 *    rounded fp32 division and square root.
 *
 * Ownership: the caller allocates and owns all device memory (the workspace,
 * x0, gradients, destinations).  The library allocates no device memory; it
 * owns only the host handle.  The workspace must stay valid until
 * ob_adam_destroy.  A handle is not thread-safe.
 *
 * Alignment: gradients are aligned to their element size (4 bytes fp32, 2
 * bytes bf16), get/set buffers to the field's element size (8 bytes for sign
 * words, else 4); OB_ERR_ARG otherwise.
 *
 * Streams: every call is enqueued on the stream given to ob_adam_init (a
 * hipStream_t passed as void*; NULL = the null stream) and returns without
 * waiting, except where stated.  Gradients must stay valid until the stream
 * has passed the call.
 *
 * Errors: argument, shape and phase errors return before anything is
 * enqueued and leave the state untouched.  A HIP launch error returns
 * OB_ERR_HIP and poisons the handle (later calls return OB_ERR_HIP).
 * Faults inside kernels surface at the next synchronizing call.  No C++
 * exception crosses this interface.
 */
#ifndef OB_ADAM_H
#define OB_ADAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ob_adam_handle* ob_adam_t;

typedef enum {
  OB_OK = 0,
  OB_ERR_ARG = 1,       /* null or misaligned pointer, bad dtype, bad worker index, bad range */
  OB_ERR_SHAPE = 2,     /* d, n do not satisfy the shape rule */
  OB_ERR_PHASE = 3,     /* call out of order (see each entry point) */
  OB_ERR_WORKSPACE = 4, /* workspace too small or misaligned */
  OB_ERR_HIP = 5,       /* HIP runtime error; the handle is poisoned */
  OB_ERR_TOO_LARGE = 6  /* the step's scratch exceeds the static scratch (see
                           ob_adam_compressed_step_static) */
} ob_status;

/* Gradient element types. */
enum { OB_GRAD_F32 = 0, OB_GRAD_BF16 = 1 };

/* Compression-phase method of a handle: 1-bit Adam (ob_adam_compressed_step
 * and its variants) or the 0/1 Adam variant (ob_adam_zero_one_step). */
enum { OB_METHOD_ONE_BIT = 0, OB_METHOD_ZERO_ONE = 1 };

typedef struct {
  int64_t d;          /* parameters; 0 < d <= 2^40, d % (64*n_workers) == 0 and
                         d / n_workers <= 2^30 (chunk length; <= 2^28 for 32
                         and 64 workers) */
  int32_t n_workers;  /* simulated workers; 1 <= n_workers <= 64 */
  int32_t grad_dtype; /* OB_GRAD_F32 or OB_GRAD_BF16 (bf16 is widened exactly) */
  float beta1, beta2, eps;
  int32_t method;     /* OB_METHOD_ONE_BIT (0, also what a zero-filled or
                         six-member initializer gives) or OB_METHOD_ZERO_ONE,
                         which reserves two more fp32 slabs per worker */
} ob_adam_config;

/* Fields for ob_adam_get_state / ob_adam_set_state. */
enum {
  OB_X = 0,            /* fp32[d] parameters */
  OB_M = 1,            /* fp32[d] momentum (after a compressed step: the decompressed server output) */
  OB_V = 2,            /* fp32[d] variance (frozen in the compression phase) */
  OB_E_WORKER = 3,     /* fp32[d] error of worker `worker` */
  OB_E_SERVER = 4,     /* fp32[d] server error */
  OB_BITS_WORKER = 5,  /* uint64[d/64] last sign words of worker `worker` */
  OB_BITS_SERVER = 6,  /* uint64[d/64] last server sign words */
  OB_SCALE_WORKER = 7, /* fp32[n] last scales of worker `worker`, one per chunk */
  OB_SCALE_SERVER = 8, /* fp32[n] last server scales, one per chunk */
  /* 0/1 Adam handles only (OB_ERR_ARG otherwise): */
  OB_M_LOCAL = 9,      /* fp32[d] local momentum of worker `worker` in the open
                          local period (OB_ERR_PHASE right after a sync) */
  OB_A_LOCAL = 10,     /* fp32[d] its step-size-weighted mean momentum over the
                          period (OB_ERR_PHASE right after a sync) */
  OB_X_LOCAL = 11      /* fp32[d] its local model: x - G*(a/(sqrtf(v)+eps)) with G
                          the period's summed step sizes; x right after a sync */
};

/* Bytes of device workspace a configuration needs (256-byte aligned start). */
ob_status ob_adam_workspace_bytes(const ob_adam_config* cfg, uint64_t* bytes);

/* Carve the state out of `workspace` (device memory, ws_bytes long, 256-byte
 * aligned) and set x = x0 (device fp32[d]; NULL = zeros), m = v = errors = 0,
 * step counter 0.  The copy and the clears are enqueued on `stream`. */
ob_status ob_adam_init(const ob_adam_config* cfg, void* workspace, uint64_t ws_bytes,
                       const float* x0, void* stream, ob_adam_t* out);

/* One full-precision Adam step on the average of the n gradients (the
 * warm-up of the method; "1-bit Adam ..." Abstract; "LIT-278" Key takeaways,
 * empirical result).  grads: host array of n device pointers, each d
 * elements of cfg.grad_dtype.  lr: this step's learning rate.
 * OB_ERR_PHASE after any compressed step. */
ob_status ob_adam_warmup_step(ob_adam_t h, const void* const* grads, float lr);

/* The same warm-up step with the gradients supplied one worker at a time
 * (bounded memory: a caller can regenerate each worker's gradient into one
 * buffer).  Call ob_adam_warmup_worker for workers 0, 1, ..., n-1 in that
 * order (`grad` is d device elements of cfg.grad_dtype and may be reused
 * once the call's work has passed on the stream), then ob_adam_warmup_finish.
 * The partial sums are kept in the workspace (in the worker error slabs,
 * which are zero throughout the warm-up and are cleared again by the finish)
 * and grouped exactly as the pairwise-by-levels sum, so results are identical
 * to ob_adam_warmup_step.  OB_ERR_PHASE for a worker out of order, for finish
 * before all n workers, after any compressed step, and for the other step
 * calls while such a step is open. */
ob_status ob_adam_warmup_worker(ob_adam_t h, int32_t worker, const void* grad);
ob_status ob_adam_warmup_finish(ob_adam_t h, float lr);

/* One compression-phase step (the contract above), all n workers at once.
 * grads as for ob_adam_warmup_step.  OB_ERR_PHASE before any warm-up step or
 * while a staged step is open.  The variance is the one left by the last
 * warm-up step and is never written again.
 * The call enqueues kernel launches only (no allocation, no memset, no wait
 * for the stream unless debug mode is on), so a caller may capture it in a
 * HIP graph on the handle's stream, after the first compressed step (which
 * reads the warm-up's fp32 momentum); each replay is one more step with the
 * captured gradients' addresses and lr.  The step counters count calls, so
 * replays are not counted. */
ob_status ob_adam_compressed_step(ob_adam_t h, const void* const* grads, float lr);

/* The same step as ob_adam_compressed_step, for callers that cannot
 * allocate device memory, or let anything allocate it, while they step (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): it allocates nothing (no hipMalloc, hipFree or allocating
 * library routine) and keeps the step's scratch -- the fixed-order partial
 * sums of squares of the workers and of the server and the finalize's group
 * results -- in a static array of the library's device code, 32 MiB per GPU,
 * instead of in the workspace (whose own scratch region it leaves alone).
 * The library's device code holds that array on every GPU it is loaded on
 * until the process ends; its device address is looked up (once per GPU)
 * on the first call on that GPU.  Results are identical to
 * ob_adam_compressed_step (the same kernels).
 *  - OB_ERR_TOO_LARGE, before anything is enqueued, when the configuration's
 *    scratch exceeds 32 MiB (8 bytes per partial: n*n worker rows of
 *    ceil(L/4096) partials, n server rows of ceil(L/4096) -- ceil(L/1024)
 *    with 32 or 64 workers -- plus the group results of rows longer than
 *    16384 partials; e.g. 1.56e9 params over 8 workers need 27 MiB);
 *  - OB_ERR_ARG when the current device is not the workspace's;
 *  - otherwise the errors and phase rules of ob_adam_compressed_step.
 * Every call on one GPU shares that GPU's array, which keeps whatever the
 * last call left there (nothing in it needs to start at zero: each step
 * writes every partial before reading it).  Calls that overlap on one GPU
 * -- two handles stepping on different streams at once -- race on the
 * array: order them (one stream, or events). */
ob_status ob_adam_compressed_step_static(ob_adam_t h, const void* const* grads, float lr);

/* One step of the 0/1 Adam variant ("Maximizing Communication Efficiency for
 * Large-scale Training via 0/1 Adam", abstract: each Adam step is made
 * linear by stale state estimates and the linear correlation of momentum and
 * update, so 1-bit compression and local steps combine), for handles made
 * with method OB_METHOD_ZERO_ONE, in the compression phase (after at least
 * one warm-up step; OB_ERR_PHASE otherwise, and for 1-bit handles).
 * Per worker i and element (fp32, in this order):
 *  - G = lr at the first step of a local period, G + lr after; w = lr / G;
 *  - m_i = (b1*m_src) + ((1-b1)*g_i), m_src = the shared momentum at the
 *    period's first step, m_i after;
 *  - a_i = m_i at the first step, a_i + (w*(m_i - a_i)) after (the
 *    step-weighted mean momentum; the worker's local model is
 *    x - G*(a_i/(sqrtf(v)+eps)), linear in its gradients while v is stale).
 * flags & OB_ZO_SYNC closes the period: c_i = a_i + e_i goes through the
 * compressed step's codec (per-chunk scale, sign words, worker error; server
 * average, server error, server scale and words), the decompressed server
 * output becomes the shared momentum m, and x = x - G*(m/(sqrtf(v)+eps)).
 * flags & OB_ZO_REFRESH (only with OB_ZO_SYNC; OB_ERR_ARG otherwise) then
 * refreshes the stale variance: v = (b2*v) + ((1-b2)*(gbar*gbar)), gbar the
 * pairwise worker average of this step's gradients as in the warm-up.
 * With OB_ZO_SYNC at every step and no refresh the result equals
 * ob_adam_compressed_step's bit for bit.  grads as for that call.  The
 * schedule of synchronizations and refreshes is the caller's.  Counters
 * (ob_adam_get_counters) can be taken only between local periods. */
enum { OB_ZO_SYNC = 1, OB_ZO_REFRESH = 2 };
ob_status ob_adam_zero_one_step(ob_adam_t h, const void* const* grads, float lr, int32_t flags);

/* The same step with the gradients supplied one worker at a time, so that a
 * caller can regenerate each worker's gradient into one buffer (bounded
 * memory).  Call ob_adam_compress_worker once for every worker w (any order;
 * `grad` is d device elements and may be reused after the call's work has
 * passed on the stream), then ob_adam_compressed_finish.  Results are
 * identical to ob_adam_compressed_step.  OB_ERR_PHASE for a worker given twice
 * in one step, for finish before all workers, and before any warm-up step. */
ob_status ob_adam_compress_worker(ob_adam_t h, int32_t worker, const void* grad);
ob_status ob_adam_compressed_finish(ob_adam_t h, float lr);

/* Copy `count` elements starting at element `offset` of a field (for
 * OB_E_WORKER, OB_BITS_WORKER and OB_SCALE_WORKER of worker `worker`) into
 * device memory `dst_device`.  Derived fields (errors, decompressed momentum)
 * are materialized by a kernel.  Enqueued on the handle's stream; the range
 * must lie inside the field (OB_ERR_ARG otherwise).
 * The destination is device memory and the call does not wait: a field of
 * the large configurations is gigabytes, so the library neither stages it
 * through host memory nor stalls the stream; a caller that wants it on the
 * host copies the device buffer afterwards (the Python binding's get() returns
 * a device tensor).  The step counter and the phase are not fields here:
 * ob_adam_get_counters returns the steps taken, the compressed steps and the
 * warm-up steps, and the phase follows from them (compression phase once a
 * compressed step was taken).   OB_E_WORKER and
 * OB_BITS_WORKER are refused (OB_ERR_PHASE) while a worker-at-a-time
 * compressed step is open, as they would mix the old and the new step, and
 * OB_E_WORKER while a worker-at-a-time warm-up step is open. */
ob_status ob_adam_get_state(ob_adam_t h, int32_t field, int32_t worker, int64_t offset,
                            int64_t count, void* dst_device);

/* Overwrite `count` elements of OB_X (always) or OB_V (only before the first
 * compressed step) from device memory (enqueued, no wait); OB_ERR_ARG for
 * other fields.  Only these two: every other field is either derived (the
 * errors from the stored compensated values and scales, the momentum from
 * the server's sign words and scales after the first compressed step) or
 * must stay consistent with the sign words and scales the next step reads,
 * and the frozen variance must not change once it preconditions compressed
 * steps.  A whole state (all fields and the counters) is restored with
 * ob_adam_attach from a copy of the workspace. */
ob_status ob_adam_set_state(ob_adam_t h, int32_t field, int64_t offset, int64_t count,
                            const void* src_device);

/* Device address of the parameters x (fp32[d], contiguous, inside the
 * caller's workspace), so that a caller can keep its parameter tensors as
 * views of it instead of copying them in and out every step.  The caller may
 * read and write x between steps, ordered on the handle's stream. */
ob_status ob_adam_params(ob_adam_t h, float** x_device);

/* Checkpoint / resume.  The whole optimizer state is the workspace bytes
 * plus these three counters (the segment partials inside the workspace are
 * scratch and may be anything).  To checkpoint: let the stream pass the last
 * step, copy ws_bytes of the workspace and read the counters.  To resume:
 * put the copy into a workspace (same config, same size, 256-byte aligned)
 * and attach it; later steps are bit-identical to an uninterrupted run. */
typedef struct {
  int64_t steps;            /* warm-up + compressed steps taken */
  int64_t compressed_steps; /* compressed steps taken */
  int64_t warmup_steps;     /* warm-up steps taken */
} ob_adam_counters;

/* OB_ERR_PHASE while a worker-at-a-time step (warm-up or compressed) or a
 * 0/1 Adam local period is open. */
ob_status ob_adam_get_counters(ob_adam_t h, ob_adam_counters* out);

/* Like ob_adam_init, but adopts a workspace that already holds a state
 * (nothing is cleared or enqueued).  OB_ERR_ARG for counters that no run
 * can produce (negative, steps != warm-up + compressed, compressed steps
 * without a warm-up step). */
ob_status ob_adam_attach(const ob_adam_config* cfg, void* workspace, uint64_t ws_bytes,
                         const ob_adam_counters* counters, void* stream, ob_adam_t* out);

/* Workspace integrity check, for debugging and tests.  Every sub-buffer of
 * the workspace is followed directly by a 256-byte guard region that
 * ob_adam_init fills with a known pattern and no kernel writes.  This call
 * synchronizes the handle's stream, reads the guards back and sets
 * *first_bad to -1 when all are intact, else to the index (in workspace
 * order: x, m, v, u, worker compensated slabs, worker sign words, server sign
 * words, worker partials, server partials, fold buffer, worker scales, server
 * scales, 0/1 local momenta, 0/1 mean momenta -- the last two empty for
 * 1-bit handles) of the first guard found changed -- a write past that buffer's
 * end.  A workspace adopted by ob_adam_attach keeps the guards of the copy. */
ob_status ob_adam_check_guards(ob_adam_t h, int32_t* first_bad);

/* Debug mode (off by default; also set at init from the environment variable
 * OB_DEBUG, read as an integer of these flags):
 *  OB_DEBUG_SYNC   - every kernel launch is followed by a wait for the
 *                    stream, so that a failing kernel is reported (on stderr,
 *                    with its OB_K_* id) by the call that launched it;
 *  OB_DEBUG_GUARDS - after every completed step the workspace guards are
 *                    checked; a changed guard is reported on stderr, the
 *                    handle is poisoned and the step returns OB_ERR_HIP;
 *  OB_DEBUG_SEPARATE_SCALES - the per-chunk scales always come from
 *                    finalize dispatches of their own.  Without it, shapes
 *                    whose chunks leave at most 64 partials per row (and n
 *                    times that at most 1024; chunks of up to 256K elements
 *                    for n <= 16) have them folded inside the server pass
 *                    and the update, in the same order: a step is then three
 *                    dispatches, and OB_K_WORKER_SCALE / OB_K_SERVER_SCALE
 *                    record no launches;
 *  OB_DEBUG_UNSTAGED_SERVER - the server pass for 8, 16, 32 and 64 workers
 *                    loads every worker's sign words of a segment straight
 *                    into registers, half a 128-byte line at a time.
 *                    Without it, chunks of an even number of 64-element rows
 *                    have each segment's words copied whole into LDS first
 *                    (gfx950's direct global-to-LDS load), so no line is
 *                    fetched twice;
 *  OB_DEBUG_SMALL_LAUNCHES - the streaming passes (worker, 0/1 local and
 *                    synchronizing, server, update) are issued as launches of
 *                    about 4096 elements each instead of about 2^26, which
 *                    exercises how a pass is cut into launches on small
 *                    shapes (a large shape would take many thousands of
 *                    launches a pass).
 * The first two make every call synchronous.  None changes a result bit.
 * OB_ERR_ARG for other flag bits. */
enum {
  OB_DEBUG_SYNC = 1,
  OB_DEBUG_GUARDS = 2,
  OB_DEBUG_SEPARATE_SCALES = 4,
  OB_DEBUG_UNSTAGED_SERVER = 8,
  OB_DEBUG_SMALL_LAUNCHES = 16
};
ob_status ob_adam_set_debug(ob_adam_t h, int32_t flags);

/* Steps taken so far (warm-up and compressed) and compressed steps taken. */
ob_status ob_adam_step_count(ob_adam_t h, int64_t* steps, int64_t* compressed_steps);

/* Kernels of a step, for ob_adam_kernel_times. */
enum {
  OB_K_WARMUP = 0,        /* warm-up Adam pass (staged: each worker's pass and the finish) */
  OB_K_WORKER = 1,        /* worker compress pass (all workers of one call) */
  OB_K_WORKER_SCALE = 2,  /* worker scale finalize */
  OB_K_SERVER = 3,        /* server average / re-compress pass */
  OB_K_SERVER_SCALE = 4,  /* server scale finalize */
  OB_K_UPDATE = 5,        /* decompress + frozen-variance update */
  OB_K_ZO_LOCAL = 6,      /* 0/1 Adam local step (a sync step's worker pass is OB_K_WORKER) */
  OB_K_ZO_REFRESH = 7,    /* 0/1 Adam variance refresh */
  OB_NUM_KERNELS = 8
};

/* Per-kernel timing.  With max_launches > 0, each later launch of an OB_K_*
 * kernel gets a pair of HIP events taken from its dispatch packets on the
 * handle's stream (the runtime's extended launch; no extra packets between
 * kernels), up to max_launches launches (later ones are counted as dropped);
 * 0 turns timing off and releases the events.  A kernel made of several
 * dispatches -- a streaming pass over more than about 2^26 elements is cut
 * into launches of that size, a long scale finalize takes two -- is timed
 * from the start of its first dispatch to the end of its last.  The events
 * are host-side runtime objects (no device memory is allocated). */
ob_status ob_adam_set_timing(ob_adam_t h, int32_t max_launches);

/* Synchronize the stream, then return for each kernel (index OB_K_*) the
 * summed event-measured duration in milliseconds and the number of timed
 * launches since timing was enabled, and the number of dropped launches. */
ob_status ob_adam_kernel_times(ob_adam_t h, double* ms /* [OB_NUM_KERNELS] */,
                               int64_t* launches /* [OB_NUM_KERNELS] */, int64_t* dropped);

/* Release the host handle (the caller frees the workspace afterwards). */
ob_status ob_adam_destroy(ob_adam_t h);

/* Static description of a status code ("unknown status" for any other value). */
const char* ob_status_str(ob_status s);

#ifdef __cplusplus
}
#endif
#endif
