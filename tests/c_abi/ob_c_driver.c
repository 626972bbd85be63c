/* A plain C caller of the ob_adam C interface (no Python, no torch): device
 * memory from hipMalloc, warm-up and compressed steps, the state read back
 * with ob_adam_get_state and compared with the CPU oracle, which is linked
 * in as test infrastructure.  Also checks a few error paths and the
 * workspace guards.  A second handle with the 0/1 Adam method runs local
 * steps, synchronizations and a variance refresh; its fields, the open
 * period's local ones included, must equal the oracle's bit for bit.
 *
 * usage: ob_c_driver d n        exit status 0 = every check passed
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ob_adam.h"
#include "ob_oracle.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      exit(2);                                                              \
    }                                                                       \
  } while (0)
#define OB_OK_(call)                                                        \
  do {                                                                      \
    ob_status s_ = (call);                                                  \
    if (s_ != OB_OK) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #call, ob_status_str(s_));         \
      exit(3);                                                              \
    }                                                                       \
  } while (0)

static int failures = 0;

static void check(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

/* xorshift64* test data in [-scale, scale) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float next_uniform(float scale) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  const uint64_t r = rng_state * 0x2545F4914F6CDD1Dull;
  return scale * (2.0f * (float)(r >> 40) / 16777216.0f - 1.0f);
}

/* fp32 field: |gpu - oracle| <= max(1e-5 |oracle|, 1e-6) everywhere */
static void compare_f32(ob_adam_t h, ob_oracle* o, int32_t field, int32_t ofield, int32_t worker,
                        int64_t count, float* dev, float* host, const char* what) {
  int64_t cnt = 0;
  const float* ref = (const float*)ob_oracle_field(o, ofield, worker, &cnt);
  check(ref != NULL && cnt == count, what);
  OB_OK_(ob_adam_get_state(h, field, worker, 0, count, dev));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(host, dev, sizeof(float) * (size_t)count, hipMemcpyDeviceToHost));
  for (int64_t k = 0; k < count; ++k) {
    const double g = host[k], r = ref[k];
    const double tol = fmax(1e-5 * fabs(r), 1e-6);
    if (!(fabs(g - r) <= tol)) {
      fprintf(stderr, "%s[%lld]: gpu %.9g oracle %.9g\n", what, (long long)k, g, r);
      check(0, what);
      return;
    }
  }
}

/* sign words or scale bit patterns: identical */
static void compare_bits(ob_adam_t h, ob_oracle* o, int32_t field, int32_t ofield, int32_t worker,
                         int64_t count, size_t elem, void* dev, void* host, const char* what) {
  int64_t cnt = 0;
  const void* ref = ob_oracle_field(o, ofield, worker, &cnt);
  check(ref != NULL && cnt >= count, what);
  OB_OK_(ob_adam_get_state(h, field, worker, 0, count, dev));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(host, dev, elem * (size_t)count, hipMemcpyDeviceToHost));
  check(memcmp(host, ref, elem * (size_t)count) == 0, what);
}

/* fresh test gradients for every worker, copied to the device on `stream` */
static void new_grads(int64_t d, int32_t n, float** hg, void** dg, hipStream_t stream) {
  for (int w = 0; w < n; ++w) {
    for (int64_t k = 0; k < d; ++k) hg[w][k] = next_uniform(1e-2f);
    HIP_OK(hipMemcpyAsync(dg[w], hg[w], sizeof(float) * (size_t)d, hipMemcpyHostToDevice,
                          stream));
  }
}

/* 0/1 Adam: one warm-up step, then local (L), synchronizing (S) and
 * synchronizing-with-refresh (R) steps with a step size that changes every
 * step.  While a period is open the local momentum, mean momentum and local
 * model of every worker are compared; after the last step every shared field. */
static void run_zero_one(int64_t d, int32_t n, float** hg, void** dg, float* dev, float* host,
                         hipStream_t stream) {
  static const char plan[] = "LRLLSLR";
  const int steps = (int)(sizeof(plan) - 1);
  ob_adam_config cfg = {d, n, OB_GRAD_F32, 0.9f, 0.999f, 1e-8f, OB_METHOD_ZERO_ONE};
  uint64_t bytes = 0;
  OB_OK_(ob_adam_workspace_bytes(&cfg, &bytes));
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, bytes));
  ob_adam_t h = NULL;
  OB_OK_(ob_adam_init(&cfg, ws, bytes, NULL, (void*)stream, &h));
  ob_oracle* o = ob_oracle_create(d, n, 0, n, cfg.beta1, cfg.beta2, cfg.eps, 1);
  check(o != NULL, "oracle create (0/1)");
  if (o == NULL) exit(4);

  new_grads(d, n, hg, dg, stream);
  check(ob_adam_compressed_step(h, (const void* const*)dg, 1e-3f) == OB_ERR_PHASE,
        "1-bit compressed step on a 0/1 handle");
  OB_OK_(ob_adam_warmup_step(h, (const void* const*)dg, 1e-3f));
  ob_oracle_warmup_step(o, (const void* const*)hg, 0, 1e-3f);
  HIP_OK(hipStreamSynchronize(stream));
  check(ob_adam_zero_one_step(h, (const void* const*)dg, 1e-3f, OB_ZO_REFRESH) == OB_ERR_ARG,
        "refresh without a synchronization");

  for (int t = 0; t < steps; ++t) {
    const float lr = 1e-3f * (1.0f + 0.25f * (float)(t % 3));
    const int sync = plan[t] != 'L', refresh = plan[t] == 'R';
    new_grads(d, n, hg, dg, stream);
    OB_OK_(ob_adam_zero_one_step(h, (const void* const*)dg, lr,
                                 (sync ? OB_ZO_SYNC : 0) | (refresh ? OB_ZO_REFRESH : 0)));
    ob_oracle_zo_step(o, (const void* const*)hg, 0, lr, sync, refresh);
    HIP_OK(hipStreamSynchronize(stream));
    if (!sync) {
      check(ob_oracle_zo_open(o) > 0, "oracle period open");
      for (int w = 0; w < n; ++w) {
        compare_bits(h, o, OB_M_LOCAL, OBO_M_LOCAL, w, d, 4, dev, host, "0/1 local momentum");
        compare_bits(h, o, OB_A_LOCAL, OBO_A_LOCAL, w, d, 4, dev, host, "0/1 mean momentum");
        compare_bits(h, o, OB_X_LOCAL, OBO_X_LOCAL, w, d, 4, dev, host, "0/1 local model");
      }
    } else {
      check(ob_adam_get_state(h, OB_M_LOCAL, 0, 0, d, dev) == OB_ERR_PHASE,
            "local momentum outside an open period");
    }
  }
  compare_bits(h, o, OB_X, OBO_X, 0, d, 4, dev, host, "0/1 x");
  compare_bits(h, o, OB_M, OBO_M, 0, d, 4, dev, host, "0/1 m");
  compare_bits(h, o, OB_V, OBO_V, 0, d, 4, dev, host, "0/1 v");
  compare_bits(h, o, OB_E_SERVER, OBO_E_SERVER, 0, d, 4, dev, host, "0/1 server error");
  compare_bits(h, o, OB_SCALE_SERVER, OBO_SCALE_SERVER, 0, n, 4, dev, host, "0/1 server scales");
  for (int w = 0; w < n; ++w) {
    compare_bits(h, o, OB_E_WORKER, OBO_E_WORKER, w, d, 4, dev, host, "0/1 worker error");
    compare_bits(h, o, OB_BITS_WORKER, OBO_BITS_WORKER, w, d / 64, 8, dev, host,
                 "0/1 worker sign words");
  }
  int32_t bad_guard = 0;
  OB_OK_(ob_adam_check_guards(h, &bad_guard));
  check(bad_guard == -1, "0/1 workspace guards");
  OB_OK_(ob_adam_destroy(h));
  ob_oracle_destroy(o);
  HIP_OK(hipFree(ws));
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s d n\n", argv[0]);
    return 1;
  }
  const int64_t d = atoll(argv[1]);
  const int32_t n = atoi(argv[2]);
  const int warm = 2, comp = 3;
  const float lr = 1e-3f;

  /* error paths: nothing is enqueued, no handle is made */
  ob_adam_config bad = {d + 1, n, OB_GRAD_F32, 0.9f, 0.999f, 1e-8f, OB_METHOD_ONE_BIT};
  uint64_t bytes = 0;
  check(ob_adam_workspace_bytes(&bad, &bytes) == OB_ERR_SHAPE, "shape rule");
  check(ob_adam_workspace_bytes(NULL, &bytes) == OB_ERR_ARG, "null config");
  check(ob_status_str(OB_ERR_PHASE) != NULL, "status string");

  ob_adam_config cfg = {d, n, OB_GRAD_F32, 0.9f, 0.999f, 1e-8f, OB_METHOD_ONE_BIT};
  OB_OK_(ob_adam_workspace_bytes(&cfg, &bytes));
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, bytes));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  ob_adam_t h = NULL;
  OB_OK_(ob_adam_init(&cfg, ws, bytes, NULL, (void*)stream, &h));
  ob_oracle* o = ob_oracle_create(d, n, 0, n, cfg.beta1, cfg.beta2, cfg.eps, 1);
  check(o != NULL, "oracle create");
  if (o == NULL) return 4;

  float** hg = (float**)malloc(sizeof(float*) * (size_t)n);
  void** dg = (void**)malloc(sizeof(void*) * (size_t)n);
  for (int w = 0; w < n; ++w) {
    hg[w] = (float*)malloc(sizeof(float) * (size_t)d);
    HIP_OK(hipMalloc(&dg[w], sizeof(float) * (size_t)d));
  }
  check(ob_adam_compressed_step(h, (const void* const*)dg, lr) == OB_ERR_PHASE,
        "compressed step before any warm-up step");

  for (int t = 0; t < warm + comp; ++t) {
    new_grads(d, n, hg, dg, stream);
    if (t < warm) {
      OB_OK_(ob_adam_warmup_step(h, (const void* const*)dg, lr));
      ob_oracle_warmup_step(o, (const void* const*)hg, 0, lr);
    } else {
      OB_OK_(ob_adam_compressed_step(h, (const void* const*)dg, lr));
      ob_oracle_compressed_step(o, (const void* const*)hg, 0, lr);
    }
    /* the host gradients are rewritten next step: let the copies finish */
    HIP_OK(hipStreamSynchronize(stream));
  }
  check(ob_adam_warmup_step(h, (const void* const*)dg, lr) == OB_ERR_PHASE,
        "warm-up step after a compressed step");

  int64_t steps = 0, csteps = 0;
  OB_OK_(ob_adam_step_count(h, &steps, &csteps));
  check(steps == ob_oracle_step(o) && csteps == comp, "step counter");

  float* dev = NULL;
  HIP_OK(hipMalloc((void**)&dev, sizeof(float) * (size_t)d));
  float* host = (float*)malloc(sizeof(float) * (size_t)d);
  compare_f32(h, o, OB_X, OBO_X, 0, d, dev, host, "x");
  compare_f32(h, o, OB_M, OBO_M, 0, d, dev, host, "m");
  compare_f32(h, o, OB_V, OBO_V, 0, d, dev, host, "v");
  compare_f32(h, o, OB_E_SERVER, OBO_E_SERVER, 0, d, dev, host, "server error");
  compare_bits(h, o, OB_BITS_SERVER, OBO_BITS_SERVER, 0, d / 64, 8, dev, host,
               "server sign words");
  compare_bits(h, o, OB_SCALE_SERVER, OBO_SCALE_SERVER, 0, n, 4, dev, host, "server scales");
  for (int w = 0; w < n; ++w) {
    compare_f32(h, o, OB_E_WORKER, OBO_E_WORKER, w, d, dev, host, "worker error");
    compare_bits(h, o, OB_BITS_WORKER, OBO_BITS_WORKER, w, d / 64, 8, dev, host,
                 "worker sign words");
    compare_bits(h, o, OB_SCALE_WORKER, OBO_SCALE_WORKER, w, n, 4, dev, host, "worker scales");
  }
  int32_t bad_guard = 0;
  OB_OK_(ob_adam_check_guards(h, &bad_guard));
  check(bad_guard == -1, "workspace guards");

  OB_OK_(ob_adam_destroy(h));
  ob_oracle_destroy(o);
  run_zero_one(d, n, hg, dg, dev, host, stream);
  for (int w = 0; w < n; ++w) {
    free(hg[w]);
    HIP_OK(hipFree(dg[w]));
  }
  free(hg);
  free(dg);
  free(host);
  HIP_OK(hipFree(dev));
  HIP_OK(hipFree(ws));
  HIP_OK(hipStreamDestroy(stream));
  if (failures) return 5;
  printf("c driver ok: d=%lld n=%d, %d warm-up + %d compressed steps and a 0/1 run match "
         "the oracle\n", (long long)d, n, warm, comp);
  return 0;
}
