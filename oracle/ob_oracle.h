/*
 * CPU oracle for the compression-phase step of 1-bit Adam.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, single-threaded, slow C that states the
 * method step by step.  Only the test suite, the smoke check and the CPU
 * baseline of the benchmark may load it; the product library never does, and
 * it shares no code with the HIP path.
 *
 * Sources (titles and sections of the pages this follows):
 *  - "1-bit Adam: Communication Efficient Large-Scale Training with Adam's
 *    Convergence Speed", Abstract: error-compensated 1-bit compression; Adam's
 *    variance becomes a fixed preconditioner after a warm-up phase.
 *  - "LIT-278: 1-bit Adam ..." (anthology-of-the-sota), Key takeaways:
 *    1-bit compressed momentum SGD preconditioned by the frozen variance;
 *    Theorem 1 conditions: error-compensated 1-bit compression with
 *    per-chunk scaling; the empirical result's full-precision warm-up.
 *    Tag lines SOTA-214 (error feedback, applied to the momentum) and SOTA-215
 *    (freeze the variance; compress the momentum, never the update).
 *    "What the evidence does not cover": the compressed allreduce.
 *  - "Adam: A Method for Stochastic Optimization" (listed under "Builds on"):
 *    the warm-up phase is that algorithm with bias correction.
 *  - "Maximizing Communication Efficiency for Large-scale Training via 0/1
 *    Adam" (abstract): the 0/1 Adam variant, ob_oracle_zo_step, built from the
 *    same codec with local steps and a stale variance.  Its pins: with a
 *    synchronization at every step and no refresh it equals the compressed
 *    step bit for bit; local models equal a float64 re-derivation of the
 *    sequential local steps; exact dyadic cases for the model averaging of a
 *    synchronization and for the refresh.  Its readings (refresh schedule and
 *    placement, the incremental step-weighted mean) are stated in
 *    ob_oracle.c; beyond these pins the 0/1 trajectories are parity
 *    unpinned.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of this repository):
 *  - chunk j of every worker and of the server is [j*L, (j+1)*L), L = d/n;
 *  - scale = (float)(sqrt(S)/sqrt((double)L)), S = sum of c^2 in fp64 in the
 *    fixed order of ob_oracle_chunk_sumsq below;
 *  - sign bit = (c >= 0.0f), element k -> bit k%64 of uint64 word k/64;
 *  - worker average = pairwise sum by levels (pairs (2i, 2i+1), an odd tail
 *    passes up unchanged), then '/ (float)n';
 *  - server error feedback is added after the average;
 *  - after a compressed step m is the decompressed server output;
 *  - warm-up uses bias correction, the compression phase uses raw m and the
 *    raw frozen v;
 *  - worker and server errors start at zero; the step counter is int64.
 *
 * The oracle may hold a contiguous subset of chunks [j0, j1) (every chunk is
 * independent of the others); the full vector is j0 = 0, j1 = n.
 */
#ifndef OB_ORACLE_H
#define OB_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ob_oracle ob_oracle;

/* fields for ob_oracle_field() */
enum {
  OBO_X = 0,       /* fp32[cnt] parameters */
  OBO_M = 1,       /* fp32[cnt] momentum */
  OBO_V = 2,       /* fp32[cnt] variance */
  OBO_E_WORKER = 3,/* fp32[cnt] error of worker w */
  OBO_E_SERVER = 4,/* fp32[cnt] server error */
  OBO_C_WORKER = 5,/* fp32[cnt] last compensated momentum of worker w */
  OBO_U_SERVER = 6,/* fp32[cnt] last compensated server average */
  OBO_A_SERVER = 7,/* fp32[cnt] last worker average (before server error) */
  OBO_BITS_WORKER = 8, /* uint64[words] last sign words of worker w */
  OBO_BITS_SERVER = 9, /* uint64[words] last server sign words */
  OBO_SCALE_WORKER = 10, /* fp32[nch] last scales of worker w, one per held chunk */
  OBO_SCALE_SERVER = 11, /* fp32[nch] last server scales */
  /* 0/1 Adam (after its first ob_oracle_zo_step): */
  OBO_M_LOCAL = 12,      /* fp32[cnt] local momentum of worker w */
  OBO_A_LOCAL = 13,      /* fp32[cnt] step-weighted mean momentum of worker w */
  OBO_X_LOCAL = 14       /* fp32[cnt] local model of worker w (computed on request) */
};

/* d % n must be 0; if the held range does not start at a multiple of 64 the
 * whole vector must be held (j0 = 0, j1 = n).  keep_debug = 0 keeps only the
 * optimizer state (the C, U and A fields are then unavailable), which bounds
 * memory on large configurations.  Returns NULL on bad arguments or
 * allocation failure. */
ob_oracle* ob_oracle_create(int64_t d, int32_t n, int32_t j0, int32_t j1, float beta1, float beta2,
                            float eps, int32_t keep_debug);
void ob_oracle_destroy(ob_oracle* o);

/* grads[w] points at worker w's gradient over the held range (cnt elements);
 * gdtype 0 = fp32, 1 = bf16 bit patterns (uint16). */
void ob_oracle_warmup_step(ob_oracle* o, const void* const* grads, int32_t gdtype, float lr);
void ob_oracle_compressed_step(ob_oracle* o, const void* const* grads, int32_t gdtype, float lr);

/* One step of the 0/1 Adam variant ("Maximizing Communication Efficiency for
 * Large-scale Training via 0/1 Adam", abstract), in the compression phase:
 * every worker's local momentum step and step-weighted mean momentum; with
 * `sync` the 1-bit compressed exchange of the mean momenta (error feedback on
 * both sides, as in ob_oracle_compressed_step), the shared momentum and the
 * shared model update by the local period's summed step sizes; with
 * `refresh` (only together with sync) the variance's Adam update on the
 * full-precision worker average of this step's gradients, after the model
 * update.  The readings behind each part are stated in ob_oracle.c. */
void ob_oracle_zo_step(ob_oracle* o, const void* const* grads, int32_t gdtype, float lr,
                       int32_t sync, int32_t refresh);
/* Worker w's local model into out[cnt]. */
void ob_oracle_zo_local_model(ob_oracle* o, int32_t w, float* out);
/* Sum of the step sizes of the open local period, and its steps so far. */
float ob_oracle_zo_gamma(const ob_oracle* o);
int32_t ob_oracle_zo_open(const ob_oracle* o);

/* Pointer to a field (worker selects the slab for per-worker fields) and its
 * element count; the memory belongs to the oracle. */
void* ob_oracle_field(ob_oracle* o, int32_t field, int32_t worker, int64_t* count);
int64_t ob_oracle_step(const ob_oracle* o);
int64_t ob_oracle_held(const ob_oracle* o);

/* Building blocks, exported so that tests can pin them on their own. */
double ob_oracle_chunk_sumsq(const float* c, int64_t len);
float ob_oracle_chunk_scale(double sumsq, int64_t len);
float ob_oracle_pairwise_mean(const float* vals, int32_t n);

#ifdef __cplusplus
}
#endif
#endif
