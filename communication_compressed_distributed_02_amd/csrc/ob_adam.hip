// Host side of the ob_adam C interface: validation, workspace carve-up,
// phase rules and the launch sequence of a step.  See include/ob_adam.h for
// the contract; the kernels are in ob_kernels.hip.
#include "ob_adam.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "ob_kernels.h"

namespace {

// Scratch of ob_adam_compressed_step_static: the step's fixed-order partials
// and finalize group results live here instead of in the caller's
// workspace.  One copy per GPU, held until the process ends.  Host code
// never passes `scratch` itself to a kernel (in host code the name stands
// for a host-side shadow, not a device address): static_scratch() looks up
// its device address once per device with hipGetSymbolAddress and keeps it.
constexpr uint64_t kStaticScratchBytes = uint64_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on `device` (which must be current).
hipError_t static_scratch(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace

struct ob_adam_handle {
  ob::State st{};
  char* base = nullptr;       // the caller's workspace
  ob::Layout layout{};
  hipStream_t stream = nullptr;
  int64_t steps = 0;          // warm-up + compressed steps taken
  int64_t compressed = 0;     // compressed steps taken
  int64_t warm = 0;           // warm-up steps taken
  bool staged_open = false;   // a worker-at-a-time step has started
  uint64_t staged_mask = 0;   // workers already compressed in the open step
  bool warm_open = false;     // a worker-at-a-time warm-up step has started
  int warm_next = 0;          // the next worker that step expects
  bool poisoned = false;
  int32_t debug = 0;          // OB_DEBUG_* flags
  int device = -1;            // the workspace's device, once a static-scratch step asked
  int32_t method = OB_METHOD_ONE_BIT;
  // 0/1 Adam: the open local period (steps taken and their summed step sizes)
  // and whether a synchronization has put the shared momentum into sign words
  int32_t zk = 0;
  float zgamma = 0.0f;
  bool zsynced = false;
  // per-kernel timing (events recorded around each launch when enabled)
  std::vector<hipEvent_t> ev;          // 2 per timed launch
  std::vector<int> ev_kernel;          // kernel id of each timed launch
  int64_t ev_used = 0, ev_dropped = 0;
};

namespace {

bool valid_beta(float b) { return isfinite(b) && b >= 0.0f && b < 1.0f; }

// 2^40 parameters: far beyond one GPU's memory, and small enough that no size
// computed from d and n (at most 64 * 4 * d bytes) can overflow.
constexpr int64_t kMaxParams = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t bytes) { return ((uintptr_t)p & (bytes - 1)) == 0; }

// Gradient elements are read at their natural alignment.
bool grad_aligned(const ob_adam_t h, const void* g) {
  return aligned(g, h->st.grad_bf16 ? 2 : 4);
}

constexpr int32_t kDebugFlags = OB_DEBUG_SYNC | OB_DEBUG_GUARDS | OB_DEBUG_SEPARATE_SCALES |
                                OB_DEBUG_UNSTAGED_SERVER | OB_DEBUG_SMALL_LAUNCHES;
// elements per launch of a streaming pass under OB_DEBUG_SMALL_LAUNCHES: one
// block of 4 segments, so small shapes take many launches per pass
constexpr int64_t kSmallLaunchElems = 4 * ob::kSegElems;

void set_debug_flags(ob_adam_handle* h, int32_t flags) {
  h->debug = flags;
  h->st.launch_elems = (flags & OB_DEBUG_SMALL_LAUNCHES) ? kSmallLaunchElems : 0;
}

ob_status check_config(const ob_adam_config* cfg) {
  if (cfg == nullptr) return OB_ERR_ARG;
  if (cfg->grad_dtype != OB_GRAD_F32 && cfg->grad_dtype != OB_GRAD_BF16) return OB_ERR_ARG;
  if (cfg->method != OB_METHOD_ONE_BIT && cfg->method != OB_METHOD_ZERO_ONE) return OB_ERR_ARG;
  if (!valid_beta(cfg->beta1) || !valid_beta(cfg->beta2) || !isfinite(cfg->eps) ||
      cfg->eps < 0.0f)
    return OB_ERR_ARG;
  if (cfg->d <= 0 || cfg->d > kMaxParams || cfg->n_workers < 1 ||
      cfg->n_workers > ob::kMaxWorkersPerLaunch)
    return OB_ERR_SHAPE;
  if (cfg->d % (64 * (int64_t)cfg->n_workers) != 0) return OB_ERR_SHAPE;
  const int64_t L = cfg->d / cfg->n_workers;
  const int64_t nseg = (L + ob::kSegElems - 1) / ob::kSegElems;
  if (nseg > ob::kMaxSegsPerChunk) return OB_ERR_SHAPE;
  if ((cfg->n_workers == 32 || cfg->n_workers == 64) && nseg > ob::kMaxSegsPerChunkSegPartials)
    return OB_ERR_SHAPE;
  return OB_OK;
}

ob_status fail(ob_adam_t h, hipError_t e) {
  if (e == hipSuccess) return OB_OK;
  h->poisoned = true;
  return OB_ERR_HIP;
}

ob_status usable(ob_adam_t h) {
  if (h == nullptr) return OB_ERR_ARG;
  if (h->poisoned) return OB_ERR_HIP;
  return OB_OK;
}

// Run launcher `fn(t0, t1)`, handing it a pair of timing events when timing
// is on (the events are taken from the dispatch packets themselves).
template <typename F>
hipError_t timed_launch(ob_adam_t h, int kernel, F fn) {
  const int64_t cap = (int64_t)h->ev_kernel.size();
  if (cap == 0) return fn(nullptr, nullptr);
  if (h->ev_used >= cap) {
    h->ev_dropped += 1;
    return fn(nullptr, nullptr);
  }
  const int64_t i = h->ev_used;
  hipError_t e = fn(h->ev[2 * i], h->ev[2 * i + 1]);
  if (e != hipSuccess) return e;
  h->ev_kernel[i] = kernel;
  h->ev_used = i + 1;
  return hipSuccess;
}

// The launch, then (debug mode) a wait for it, so that an error is reported
// by the call that launched the failing kernel.
template <typename F>
hipError_t timed(ob_adam_t h, int kernel, F fn) {
  hipError_t e = timed_launch(h, kernel, fn);
  if (e == hipSuccess && (h->debug & OB_DEBUG_SYNC)) {
    e = hipStreamSynchronize(h->stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess)
      fprintf(stderr, "ob_adam: kernel %d (OB_K_*) failed: %s\n", kernel, hipGetErrorString(e));
  }
  return e;
}

// Synchronize and compare every guard with its pattern; *first_bad = -1 if
// all are intact, else the first changed one.
hipError_t read_guards(ob_adam_t h, int32_t* first_bad) {
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return e;
  uint32_t words[ob::kGuardBytes / 4];
  *first_bad = -1;
  for (int i = 0; i < ob::kNumGuards; ++i) {
    e = hipMemcpy(words, h->base + h->layout.guard[i], ob::kGuardBytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    for (uint64_t k = 0; k < ob::kGuardBytes / 4; ++k) {
      if (words[k] != ob::guard_word(i)) {
        *first_bad = i;
        return hipSuccess;
      }
    }
  }
  return hipSuccess;
}

// After a completed step (debug mode): the workspace guards must be intact.
ob_status after_step(ob_adam_t h) {
  if (!(h->debug & OB_DEBUG_GUARDS)) return OB_OK;
  int32_t bad = -1;
  if (read_guards(h, &bad) != hipSuccess) return fail(h, hipErrorUnknown);
  if (bad >= 0) {
    fprintf(stderr, "ob_adam: workspace guard %d changed by step %lld\n", bad,
            (long long)h->steps);
    h->poisoned = true;
    return OB_ERR_HIP;
  }
  return OB_OK;
}

void release_events(ob_adam_t h) {
  // recorded events may still be pending on the stream: let them complete
  if (h->ev_used > 0) (void)hipStreamSynchronize(h->stream);
  for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
  h->ev.clear();
  h->ev_kernel.clear();
  h->ev_used = 0;
  h->ev_dropped = 0;
}

ob_status gather_grads(ob_adam_t h, const void* const* grads, int w0, int nw, ob::GradPtrs* g) {
  if (grads == nullptr) return OB_ERR_ARG;
  for (int i = 0; i < nw; ++i) {
    if (grads[w0 + i] == nullptr || !grad_aligned(h, grads[w0 + i])) return OB_ERR_ARG;
    g->p[i] = grads[w0 + i];
  }
  return OB_OK;
}

bool any_open(ob_adam_t h) { return h->staged_open || h->warm_open; }

// Bias corrections (float)(1 - b^t) with b^t formed by t fp64 multiplications.
void bias_corrections(const ob::State& s, int64_t t, float* bc1, float* bc2) {
  double p1 = 1.0, p2 = 1.0;
  for (int64_t i = 0; i < t; ++i) {
    p1 = p1 * (double)s.beta1;
    p2 = p2 * (double)s.beta2;
  }
  *bc1 = (float)(1.0 - p1);
  *bc2 = (float)(1.0 - p2);
}

// After the worker pass(es) of a compressed or synchronizing step: worker
// scales, server pass, server scales, update with step size `lr` on state
// `s` (the handle's, or the handle's with its scratch elsewhere).  Short rows
// of partials have their scales folded inside the server pass and the
// update (three dispatches a step) unless OB_DEBUG_SEPARATE_SCALES asks for
// the finalize dispatches; OB_DEBUG_UNSTAGED_SERVER keeps the server pass's
// sign words out of LDS.
hipError_t server_and_update(ob_adam_t h, const ob::State& s, float lr) {
  hipStream_t st = h->stream;
  const bool fold = !(h->debug & OB_DEBUG_SEPARATE_SCALES) && ob::scales_in_consumers(s);
  hipError_t e = hipSuccess;
  if (!fold)
    e = timed(h, OB_K_WORKER_SCALE, [&](hipEvent_t a, hipEvent_t b) {
      return ob::launch_worker_scales(s, st, a, b);
    });
  if (e == hipSuccess)
    e = timed(h, OB_K_SERVER, [&](hipEvent_t a, hipEvent_t b) {
      return ob::launch_server_pass(s, fold, !(h->debug & OB_DEBUG_UNSTAGED_SERVER), st, a, b);
    });
  if (e == hipSuccess && !fold)
    e = timed(h, OB_K_SERVER_SCALE,
              [&](hipEvent_t a, hipEvent_t b) { return ob::launch_server_scales(s, st, a, b); });
  if (e == hipSuccess)
    e = timed(h, OB_K_UPDATE,
              [&](hipEvent_t a, hipEvent_t b) { return ob::launch_update(s, lr, fold, st, a, b); });
  return e;
}

// The rest of a compressed step after its worker pass(es); then count it.
ob_status finish_step(ob_adam_t h, const ob::State& s, float lr) {
  const hipError_t e = server_and_update(h, s, lr);
  if (e != hipSuccess) return fail(h, e);
  h->steps += 1;
  h->compressed += 1;
  return after_step(h);
}

}  // namespace

extern "C" {

ob_status ob_adam_workspace_bytes(const ob_adam_config* cfg, uint64_t* bytes) {
  ob_status st = check_config(cfg);
  if (st != OB_OK) return st;
  if (bytes == nullptr) return OB_ERR_ARG;
  *bytes = ob::layout_for(cfg->d, cfg->n_workers, cfg->method == OB_METHOD_ZERO_ONE).total;
  return OB_OK;
}

namespace {

// A handle over `workspace` (validated by the caller); nullptr if out of memory.
ob_adam_handle* make_handle(const ob_adam_config* cfg, void* workspace, void* stream) {
  const ob::Layout l = ob::layout_for(cfg->d, cfg->n_workers, cfg->method == OB_METHOD_ZERO_ONE);
  ob_adam_handle* h = new (std::nothrow) ob_adam_handle();
  if (h == nullptr) return nullptr;
  char* base = (char*)workspace;
  h->base = base;
  h->layout = l;
  ob::State& s = h->st;
  s.d = cfg->d;
  s.n = cfg->n_workers;
  s.L = cfg->d / cfg->n_workers;
  s.nseg = (s.L + ob::kSegElems - 1) / ob::kSegElems;
  s.words = cfg->d / 64;
  s.grad_bf16 = cfg->grad_dtype == OB_GRAD_BF16;
  s.beta1 = cfg->beta1;
  s.beta2 = cfg->beta2;
  s.eps = cfg->eps;
  s.x = (float*)(base + l.x);
  s.m = (float*)(base + l.m);
  s.v = (float*)(base + l.v);
  s.u = (float*)(base + l.u);
  s.c = (float*)(base + l.c);
  s.wbits = (uint64_t*)(base + l.wbits);
  s.sbits = (uint64_t*)(base + l.sbits);
  s.wpart = (double*)(base + l.wpart);
  s.spart = (double*)(base + l.spart);
  s.fold = (double*)(base + l.fold);
  s.wscale = (float*)(base + l.wscale);
  s.sscale = (float*)(base + l.sscale);
  h->method = cfg->method;
  if (cfg->method == OB_METHOD_ZERO_ONE) {
    s.mloc = (float*)(base + l.mloc);
    s.aloc = (float*)(base + l.aloc);
  }
  h->stream = (hipStream_t)stream;
  const char* dbg = getenv("OB_DEBUG");
  if (dbg != nullptr) set_debug_flags(h, atoi(dbg) & kDebugFlags);
  return h;
}

ob_status check_workspace(const ob_adam_config* cfg, void* workspace, uint64_t ws_bytes) {
  const ob::Layout l = ob::layout_for(cfg->d, cfg->n_workers, cfg->method == OB_METHOD_ZERO_ONE);
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0 || ws_bytes < l.total)
    return OB_ERR_WORKSPACE;
  return OB_OK;
}

}  // namespace

ob_status ob_adam_init(const ob_adam_config* cfg, void* workspace, uint64_t ws_bytes,
                       const float* x0, void* stream, ob_adam_t* out) {
  ob_status st = check_config(cfg);
  if (st != OB_OK) return st;
  if (out == nullptr) return OB_ERR_ARG;
  st = check_workspace(cfg, workspace, ws_bytes);
  if (st != OB_OK) return st;
  ob_adam_handle* h = make_handle(cfg, workspace, stream);
  if (h == nullptr) return OB_ERR_ARG;
  const ob::Layout l = ob::layout_for(cfg->d, cfg->n_workers, cfg->method == OB_METHOD_ZERO_ONE);
  const ob::State& s = h->st;
  hipError_t e = hipMemsetAsync(workspace, 0, l.total, h->stream);
  for (int i = 0; i < ob::kNumGuards && e == hipSuccess; ++i)
    e = hipMemsetD32Async((hipDeviceptr_t)(h->base + l.guard[i]), (int)ob::guard_word(i),
                          ob::kGuardBytes / 4, h->stream);
  if (e == hipSuccess && x0 != nullptr)
    e = hipMemcpyAsync(s.x, x0, sizeof(float) * (size_t)s.d, hipMemcpyDeviceToDevice, h->stream);
  if (e != hipSuccess) {
    delete h;
    return OB_ERR_HIP;
  }
  *out = h;
  return OB_OK;
}

ob_status ob_adam_attach(const ob_adam_config* cfg, void* workspace, uint64_t ws_bytes,
                         const ob_adam_counters* counters, void* stream, ob_adam_t* out) {
  ob_status st = check_config(cfg);
  if (st != OB_OK) return st;
  if (out == nullptr || counters == nullptr) return OB_ERR_ARG;
  const ob_adam_counters& c = *counters;
  if (c.steps < 0 || c.compressed_steps < 0 || c.warmup_steps < 0 ||
      c.steps != c.compressed_steps + c.warmup_steps ||
      (c.compressed_steps > 0 && c.warmup_steps == 0))
    return OB_ERR_ARG;
  st = check_workspace(cfg, workspace, ws_bytes);
  if (st != OB_OK) return st;
  ob_adam_handle* h = make_handle(cfg, workspace, stream);
  if (h == nullptr) return OB_ERR_ARG;
  h->steps = c.steps;
  h->compressed = c.compressed_steps;
  h->warm = c.warmup_steps;
  // 0/1 Adam: counters are taken only between local periods, so every 0/1
  // step before the checkpoint ended with (or was) a synchronization
  h->zsynced = h->method == OB_METHOD_ZERO_ONE && c.compressed_steps > 0;
  *out = h;
  return OB_OK;
}

ob_status ob_adam_get_counters(ob_adam_t h, ob_adam_counters* out) {
  if (h == nullptr || out == nullptr) return OB_ERR_ARG;
  if (any_open(h) || h->zk > 0) return OB_ERR_PHASE;
  out->steps = h->steps;
  out->compressed_steps = h->compressed;
  out->warmup_steps = h->warm;
  return OB_OK;
}

ob_status ob_adam_warmup_step(ob_adam_t h, const void* const* grads, float lr) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  if (h->compressed > 0 || any_open(h)) return OB_ERR_PHASE;
  ob::GradPtrs g{};
  st = gather_grads(h, grads, 0, h->st.n, &g);
  if (st != OB_OK) return st;
  const int64_t t = h->steps + 1;
  float bc1, bc2;
  bias_corrections(h->st, t, &bc1, &bc2);
  st = fail(h, timed(h, OB_K_WARMUP, [&](hipEvent_t a, hipEvent_t b) {
              return ob::launch_warmup(h->st, g, lr, bc1, bc2, h->stream, a, b);
            }));
  if (st != OB_OK) return st;
  h->steps = t;
  h->warm += 1;
  return after_step(h);
}

ob_status ob_adam_warmup_worker(ob_adam_t h, int32_t worker, const void* grad) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  if (worker < 0 || worker >= h->st.n || grad == nullptr || !grad_aligned(h, grad))
    return OB_ERR_ARG;
  if (h->compressed > 0 || h->staged_open) return OB_ERR_PHASE;
  if (worker != (h->warm_open ? h->warm_next : 0)) return OB_ERR_PHASE;
  st = fail(h, timed(h, OB_K_WARMUP, [&](hipEvent_t a, hipEvent_t b) {
              return ob::launch_warmup_push(h->st, grad, worker, h->stream, a, b);
            }));
  if (st != OB_OK) return st;
  h->warm_open = true;
  h->warm_next = worker + 1;
  return OB_OK;
}

ob_status ob_adam_warmup_finish(ob_adam_t h, float lr) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  if (!h->warm_open || h->warm_next != h->st.n) return OB_ERR_PHASE;
  const int64_t t = h->steps + 1;
  float bc1, bc2;
  bias_corrections(h->st, t, &bc1, &bc2);
  st = fail(h, timed(h, OB_K_WARMUP, [&](hipEvent_t a, hipEvent_t b) {
              return ob::launch_warmup_finish(h->st, lr, bc1, bc2, h->stream, a, b);
            }));
  if (st != OB_OK) return st;
  h->warm_open = false;
  h->warm_next = 0;
  h->steps = t;
  h->warm += 1;
  return after_step(h);
}

ob_status ob_adam_compressed_step(ob_adam_t h, const void* const* grads, float lr) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  if (h->warm == 0 || any_open(h) || h->method != OB_METHOD_ONE_BIT) return OB_ERR_PHASE;
  ob::GradPtrs g{};
  st = gather_grads(h, grads, 0, h->st.n, &g);
  if (st != OB_OK) return st;
  const bool m_bits = h->compressed > 0;
  st = fail(h, timed(h, OB_K_WORKER, [&](hipEvent_t a, hipEvent_t b) {
              return ob::launch_worker_pass(h->st, g, 0, h->st.n, m_bits, h->stream, a, b);
            }));
  if (st != OB_OK) return st;
  return finish_step(h, h->st, lr);
}

ob_status ob_adam_compressed_step_static(ob_adam_t h, const void* const* grads, float lr) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  const ob::ScratchLayout sl = ob::scratch_layout(h->st.nseg, h->st.n);
  if (sl.total > kStaticScratchBytes) return OB_ERR_TOO_LARGE;
  if (h->warm == 0 || any_open(h) || h->method != OB_METHOD_ONE_BIT) return OB_ERR_PHASE;
  ob::GradPtrs g{};
  st = gather_grads(h, grads, 0, h->st.n, &g);
  if (st != OB_OK) return st;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(h, hipErrorNoDevice);
  if (h->device < 0) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, h->base) != hipSuccess) return fail(h, hipErrorUnknown);
    h->device = attr.device;
  }
  if (cur != h->device) return OB_ERR_ARG;  // the scratch must be the workspace's GPU's
  void* base = nullptr;
  if (static_scratch(cur, &base) != hipSuccess) return fail(h, hipErrorInvalidSymbol);
  ob::State s = h->st;
  s.wpart = (double*)((char*)base + sl.wpart);
  s.spart = (double*)((char*)base + sl.spart);
  s.fold = (double*)((char*)base + sl.fold);
  const bool m_bits = h->compressed > 0;
  st = fail(h, timed(h, OB_K_WORKER, [&](hipEvent_t a, hipEvent_t b) {
              return ob::launch_worker_pass(s, g, 0, s.n, m_bits, h->stream, a, b);
            }));
  if (st != OB_OK) return st;
  return finish_step(h, s, lr);
}

ob_status ob_adam_compress_worker(ob_adam_t h, int32_t worker, const void* grad) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  if (worker < 0 || worker >= h->st.n || grad == nullptr || !grad_aligned(h, grad))
    return OB_ERR_ARG;
  if (h->warm == 0 || h->warm_open || h->method != OB_METHOD_ONE_BIT) return OB_ERR_PHASE;
  const uint64_t bit = (uint64_t)1 << worker;
  if (h->staged_open && (h->staged_mask & bit)) return OB_ERR_PHASE;
  ob::GradPtrs g{};
  g.p[0] = grad;
  const bool m_bits = h->compressed > 0;
  st = fail(h, timed(h, OB_K_WORKER, [&](hipEvent_t a, hipEvent_t b) {
              return ob::launch_worker_pass(h->st, g, worker, 1, m_bits, h->stream, a, b);
            }));
  if (st != OB_OK) return st;
  h->staged_open = true;
  h->staged_mask |= bit;
  return OB_OK;
}

ob_status ob_adam_compressed_finish(ob_adam_t h, float lr) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  const uint64_t all = h->st.n == 64 ? ~(uint64_t)0 : (((uint64_t)1 << h->st.n) - 1);
  if (!h->staged_open || h->staged_mask != all) return OB_ERR_PHASE;
  st = finish_step(h, h->st, lr);  // errors here leave the handle poisoned
  h->staged_open = false;
  h->staged_mask = 0;
  return st;
}

ob_status ob_adam_zero_one_step(ob_adam_t h, const void* const* grads, float lr,
                                int32_t flags) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  if ((flags & ~(OB_ZO_SYNC | OB_ZO_REFRESH)) != 0) return OB_ERR_ARG;
  const bool sync = (flags & OB_ZO_SYNC) != 0;
  const bool refresh = (flags & OB_ZO_REFRESH) != 0;
  if (refresh && !sync) return OB_ERR_ARG;
  if (h->method != OB_METHOD_ZERO_ONE || h->warm == 0 || any_open(h)) return OB_ERR_PHASE;
  ob::GradPtrs g{};
  st = gather_grads(h, grads, 0, h->st.n, &g);
  if (st != OB_OK) return st;
  // the period's summed step sizes and this step's weight in the mean
  // momentum, in fp32 as the method states them
  const bool first = h->zk == 0;
  const float gamma = first ? lr : h->zgamma + lr;
  const float wk = lr / gamma;
  const ob::State& s = h->st;
  hipStream_t stm = h->stream;
  if (!sync) {
    st = fail(h, timed(h, OB_K_ZO_LOCAL, [&](hipEvent_t a, hipEvent_t b) {
                return ob::launch_zo_local(s, g, first, h->zsynced, wk, stm, a, b);
              }));
    if (st != OB_OK) return st;
    h->zk += 1;
    h->zgamma = gamma;
  } else {
    hipError_t e = timed(h, OB_K_WORKER, [&](hipEvent_t a, hipEvent_t b) {
      return ob::launch_zo_sync(s, g, first, h->zsynced, wk, stm, a, b);
    });
    if (e == hipSuccess)  // the shared model takes the whole period's steps
      e = server_and_update(h, s, gamma);
    if (e == hipSuccess && refresh)  // after the update, which used the stale variance
      e = timed(h, OB_K_ZO_REFRESH,
                [&](hipEvent_t a, hipEvent_t b) { return ob::launch_zo_refresh(s, g, stm, a, b); });
    if (e != hipSuccess) return fail(h, e);
    h->zk = 0;
    h->zgamma = 0.0f;
    h->zsynced = true;
  }
  h->steps += 1;
  h->compressed += 1;
  return after_step(h);
}

ob_status ob_adam_get_state(ob_adam_t h, int32_t field, int32_t worker, int64_t offset,
                            int64_t count, void* dst_device) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  const ob::State& s = h->st;
  const bool zo_field = field == OB_M_LOCAL || field == OB_A_LOCAL || field == OB_X_LOCAL;
  if (zo_field && h->method != OB_METHOD_ZERO_ONE) return OB_ERR_ARG;
  // the local momenta are the open local period's (none right after a sync)
  if ((field == OB_M_LOCAL || field == OB_A_LOCAL) && h->zk == 0) return OB_ERR_PHASE;
  const bool per_worker = field == OB_E_WORKER || field == OB_BITS_WORKER ||
                          field == OB_SCALE_WORKER || zo_field;
  if (per_worker && (worker < 0 || worker >= s.n)) return OB_ERR_ARG;
  // mid-way through a worker-at-a-time step the compressed workers' slabs
  // already belong to the new step while the scales still belong to the old
  if (h->staged_open && (field == OB_E_WORKER || field == OB_BITS_WORKER)) return OB_ERR_PHASE;
  // mid-way through a worker-at-a-time warm-up step the compensated slabs
  // hold that step's partial gradient sums
  if (h->warm_open && field == OB_E_WORKER) return OB_ERR_PHASE;
  int64_t size;
  switch (field) {
    case OB_X: case OB_M: case OB_V: case OB_E_WORKER: case OB_E_SERVER:
    case OB_M_LOCAL: case OB_A_LOCAL: case OB_X_LOCAL:
      size = s.d;
      break;
    case OB_BITS_WORKER: case OB_BITS_SERVER: size = s.words; break;
    case OB_SCALE_WORKER: case OB_SCALE_SERVER: size = s.n; break;
    default: return OB_ERR_ARG;
  }
  if (offset < 0 || count < 0 || offset > size || count > size - offset) return OB_ERR_ARG;
  if (count == 0) return OB_OK;
  if (dst_device == nullptr) return OB_ERR_ARG;
  const bool words = field == OB_BITS_WORKER || field == OB_BITS_SERVER;
  if (!aligned(dst_device, words ? 8 : 4)) return OB_ERR_ARG;
  hipError_t e = hipSuccess;
  auto copy = [&](const void* src, size_t elem) {
    return hipMemcpyAsync(dst_device, (const char*)src + elem * (size_t)offset,
                          elem * (size_t)count, hipMemcpyDeviceToDevice, h->stream);
  };
  const int64_t w = worker;
  switch (field) {
    case OB_X: e = copy(s.x, 4); break;
    case OB_V: e = copy(s.v, 4); break;
    case OB_M:
      if (h->method == OB_METHOD_ZERO_ONE ? h->zsynced : h->compressed > 0)
        e = ob::launch_decompress_out(s.sbits, s.sscale, s.L, offset, count, (float*)dst_device,
                                      h->stream);
      else
        e = copy(s.m, 4);
      break;
    case OB_E_WORKER:
      e = ob::launch_error_out(s.c + w * s.d, s.wscale + w * s.n, s.L, offset, count,
                               (float*)dst_device, h->stream);
      break;
    case OB_E_SERVER:
      e = ob::launch_error_out(s.u, s.sscale, s.L, offset, count, (float*)dst_device, h->stream);
      break;
    case OB_BITS_WORKER: e = copy(s.wbits + w * s.words, 8); break;
    case OB_BITS_SERVER: e = copy(s.sbits, 8); break;
    case OB_SCALE_WORKER: e = copy(s.wscale + w * s.n, 4); break;
    case OB_SCALE_SERVER: e = copy(s.sscale, 4); break;
    case OB_M_LOCAL: e = copy(s.mloc + w * s.d, 4); break;
    case OB_A_LOCAL: e = copy(s.aloc + w * s.d, 4); break;
    case OB_X_LOCAL:
      if (h->zk == 0)
        e = copy(s.x, 4);
      else
        e = ob::launch_zo_local_model(s.x, s.aloc + w * s.d, s.v, h->zgamma, s.eps, offset, count,
                                      (float*)dst_device, h->stream);
      break;
  }
  return fail(h, e);
}

ob_status ob_adam_set_state(ob_adam_t h, int32_t field, int64_t offset, int64_t count,
                            const void* src_device) {
  ob_status st = usable(h);
  if (st != OB_OK) return st;
  const ob::State& s = h->st;
  float* dst;
  if (field == OB_X) {
    dst = s.x;
  } else if (field == OB_V) {
    if (h->compressed > 0 || any_open(h)) return OB_ERR_PHASE;
    dst = s.v;
  } else {
    return OB_ERR_ARG;
  }
  if (offset < 0 || count < 0 || offset > s.d || count > s.d - offset) return OB_ERR_ARG;
  if (count == 0) return OB_OK;
  if (src_device == nullptr || !aligned(src_device, 4)) return OB_ERR_ARG;
  return fail(h, hipMemcpyAsync(dst + offset, src_device, sizeof(float) * (size_t)count,
                                hipMemcpyDeviceToDevice, h->stream));
}

ob_status ob_adam_check_guards(ob_adam_t h, int32_t* first_bad) {
  if (h == nullptr || first_bad == nullptr) return OB_ERR_ARG;
  if (h->poisoned) return OB_ERR_HIP;
  if (read_guards(h, first_bad) != hipSuccess) return fail(h, hipErrorUnknown);
  return OB_OK;
}

ob_status ob_adam_set_debug(ob_adam_t h, int32_t flags) {
  if (h == nullptr || (flags & ~kDebugFlags) != 0) return OB_ERR_ARG;
  set_debug_flags(h, flags);
  return OB_OK;
}

ob_status ob_adam_params(ob_adam_t h, float** x_device) {
  if (h == nullptr || x_device == nullptr) return OB_ERR_ARG;
  *x_device = h->st.x;
  return OB_OK;
}

ob_status ob_adam_step_count(ob_adam_t h, int64_t* steps, int64_t* compressed_steps) {
  if (h == nullptr || steps == nullptr || compressed_steps == nullptr) return OB_ERR_ARG;
  *steps = h->steps;
  *compressed_steps = h->compressed;
  return OB_OK;
}

ob_status ob_adam_set_timing(ob_adam_t h, int32_t max_launches) {
  if (h == nullptr || max_launches < 0) return OB_ERR_ARG;
  if (h->poisoned) return OB_ERR_HIP;
  release_events(h);
  if (max_launches == 0) return OB_OK;
  h->ev.assign(2 * (size_t)max_launches, nullptr);
  for (size_t i = 0; i < h->ev.size(); ++i) {
    if (hipEventCreate(&h->ev[i]) != hipSuccess) {
      h->ev.resize(i);
      release_events(h);
      return OB_ERR_HIP;
    }
  }
  h->ev_kernel.assign((size_t)max_launches, -1);
  return OB_OK;
}

ob_status ob_adam_kernel_times(ob_adam_t h, double* ms, int64_t* launches, int64_t* dropped) {
  if (h == nullptr || ms == nullptr || launches == nullptr || dropped == nullptr)
    return OB_ERR_ARG;
  if (h->poisoned) return OB_ERR_HIP;
  for (int k = 0; k < OB_NUM_KERNELS; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  *dropped = h->ev_dropped;
  if (h->ev_used == 0) return OB_OK;
  if (hipStreamSynchronize(h->stream) != hipSuccess) return fail(h, hipErrorUnknown);
  for (int64_t i = 0; i < h->ev_used; ++i) {
    float t = 0.0f;
    if (hipEventElapsedTime(&t, h->ev[2 * i], h->ev[2 * i + 1]) != hipSuccess)
      return fail(h, hipErrorUnknown);
    ms[h->ev_kernel[i]] += (double)t;
    launches[h->ev_kernel[i]] += 1;
  }
  return OB_OK;
}

ob_status ob_adam_destroy(ob_adam_t h) {
  if (h == nullptr) return OB_ERR_ARG;
  release_events(h);
  delete h;
  return OB_OK;
}

const char* ob_status_str(ob_status s) {
  // A C caller may pass any int: read the argument's bits as an int, since
  // loading an out-of-range value through the enum type is undefined in C++.
  static_assert(sizeof(ob_status) == sizeof(int), "ob_status is an int-sized enum");
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case OB_OK: return "ok";
    case OB_ERR_ARG: return "invalid argument";
    case OB_ERR_SHAPE:
      return "unsupported shape (need 0 < d <= 2^40, 1 <= n <= 64, d % (64*n) == 0, d/n <= 2^30, "
             "and d/n <= 2^28 for n = 32 or 64)";
    case OB_ERR_PHASE: return "call out of order for the current phase";
    case OB_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case OB_ERR_HIP: return "HIP runtime error (handle poisoned)";
    case OB_ERR_TOO_LARGE:
      return "the step's scratch exceeds the library's static scratch (32 MiB per GPU)";
  }
  return "unknown status";
}

}  // extern "C"
