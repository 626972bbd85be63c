/*
 * CPU oracle for the compression-phase step of 1-bit Adam.
 * TEST INFRASTRUCTURE ONLY (see ob_oracle.h for what it follows and who may
 * use it).  Build: gcc -O2 -ffp-contract=off, no fast-math, no FTZ/DAZ.
 *
 * Every floating-point operation below is written in the order it is meant
 * to round; parentheses bind as written.
 */
#include "ob_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

struct ob_oracle {
  int64_t d;
  int32_t n;
  int64_t L;      /* chunk length d/n */
  int32_t j0, j1; /* held chunks [j0, j1) */
  int32_t nch;    /* j1 - j0 */
  int64_t cnt;    /* held elements nch*L */
  int64_t words;  /* sign words over the held range */
  float beta1, beta2, eps;
  int64_t t;
  int32_t keep_debug;

  float *x, *m, *v, *e_srv; /* [cnt] */
  float *e;                 /* [n][cnt] */
  float *c;                 /* [n][cnt] if keep_debug, else [L] scratch */
  float *u, *a;             /* [cnt] if keep_debug, else [L] scratch */
  uint64_t *wbits;          /* [n][words] */
  uint64_t *sbits;          /* [words] */
  float *wscale;            /* [n][nch] */
  float *sscale;            /* [nch] */
  float *vals;              /* [n] scratch for the worker average */

  /* 0/1 Adam (ob_oracle_zo_step), allocated on its first step */
  float *mloc;              /* [n][cnt] each worker's local momentum */
  float *aloc;              /* [n][cnt] each worker's step-weighted mean momentum */
  float *xloc;              /* [cnt] scratch: one worker's local model */
  float zgamma;             /* sum of the step sizes of the open local period */
  int32_t zk;               /* local steps taken in the open period */
};

static float grad_at(const void* g, int32_t gdtype, int64_t k) {
  if (gdtype == 0) return ((const float*)g)[k];
  /* bf16 -> fp32 is exact: the 16 bits become the top half of the fp32 word */
  union { uint32_t u; float f; } cv;
  cv.u = (uint32_t)((const uint16_t*)g)[k] << 16;
  return cv.f;
}

static void set_bit(uint64_t* words, int64_t k, int bit) {
  if (bit) words[k >> 6] |= (uint64_t)1 << (k & 63);
}

static int get_bit(const uint64_t* words, int64_t k) {
  return (int)((words[k >> 6] >> (k & 63)) & 1u);
}

/* Sum of squares of one chunk in fp64 in a fixed order (the same order any
 * implementation must use to reproduce the scale bit for bit):
 *  - the chunk is cut into segments of 1024 elements (the last may be short);
 *  - in segment s, accumulator k (k = 0..63) adds, for r = 0..15 in turn, the
 *    square of element 1024*s + 64*r + k (elements past the end add nothing);
 *  - the 64 accumulators are combined by an xor butterfly: for o = 32, 16,
 *    8, 4, 2, 1 every accumulator k becomes acc[k] + acc[k ^ o]; the segment
 *    partial is the (common) result;
 *  - the segment partials, padded with zeros to a power-of-two count, are
 *    summed pairwise level by level: p[i] = p[2i] + p[2i+1].
 * Squares of fp32 values are exact in fp64. */
double ob_oracle_chunk_sumsq(const float* c, int64_t len) {
  if (len <= 0) return 0.0;
  int64_t nseg = (len + 1023) / 1024;
  int64_t width = 1;
  while (width < nseg) width *= 2;
  double* p = (double*)calloc((size_t)width, sizeof(double));
  if (!p) abort();
  for (int64_t s = 0; s < nseg; ++s) {
    double acc[64];
    for (int k = 0; k < 64; ++k) acc[k] = 0.0;
    for (int r = 0; r < 16; ++r) {
      for (int k = 0; k < 64; ++k) {
        int64_t q = 1024 * s + 64 * r + k;
        if (q < len) {
          double cd = (double)c[q];
          acc[k] = acc[k] + cd * cd;
        }
      }
    }
    for (int o = 32; o >= 1; o /= 2) {
      double nxt[64];
      for (int k = 0; k < 64; ++k) nxt[k] = acc[k] + acc[k ^ o];
      for (int k = 0; k < 64; ++k) acc[k] = nxt[k];
    }
    p[s] = acc[0];
  }
  for (int64_t w = width; w > 1; w /= 2)
    for (int64_t i = 0; i < w / 2; ++i) p[i] = p[2 * i] + p[2 * i + 1];
  double S = p[0];
  free(p);
  return S;
}

/* Per-chunk scale: the chunk's L2 norm divided by the square root of its
 * length, computed in fp64 and rounded once to fp32. */
float ob_oracle_chunk_scale(double sumsq, int64_t len) {
  return (float)(sqrt(sumsq) / sqrt((double)len));
}

/* Mean over workers: pairwise sum by levels (pairs (2i, 2i+1); an odd last
 * element passes up unchanged), then division by n in fp32. */
float ob_oracle_pairwise_mean(const float* vals, int32_t n) {
  float tmp[4096];
  float* t = n <= 4096 ? tmp : (float*)malloc(sizeof(float) * (size_t)n);
  if (!t) abort();
  for (int32_t i = 0; i < n; ++i) t[i] = vals[i];
  int32_t cnt = n;
  while (cnt > 1) {
    int32_t half = cnt / 2;
    for (int32_t i = 0; i < half; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    if (cnt & 1) {
      t[half] = t[cnt - 1];
      cnt = half + 1;
    } else {
      cnt = half;
    }
  }
  float r = t[0] / (float)n;
  if (t != tmp) free(t);
  return r;
}

ob_oracle* ob_oracle_create(int64_t d, int32_t n, int32_t j0, int32_t j1, float beta1, float beta2,
                            float eps, int32_t keep_debug) {
  if (d <= 0 || n <= 0 || d % n != 0 || j0 < 0 || j1 > n || j0 >= j1) return NULL;
  int64_t L = d / n;
  if ((j0 * L) % 64 != 0 && !(j0 == 0 && j1 == n)) return NULL;
  ob_oracle* o = (ob_oracle*)calloc(1, sizeof(ob_oracle));
  if (!o) return NULL;
  o->d = d;
  o->n = n;
  o->L = L;
  o->j0 = j0;
  o->j1 = j1;
  o->nch = j1 - j0;
  o->cnt = (int64_t)o->nch * L;
  o->words = (o->cnt + 63) / 64;
  o->beta1 = beta1;
  o->beta2 = beta2;
  o->eps = eps;
  o->t = 0;
  o->keep_debug = keep_debug;
  size_t cnt = (size_t)o->cnt;
  size_t dbg = keep_debug ? cnt : (size_t)L;
  o->x = (float*)calloc(cnt, sizeof(float));
  o->m = (float*)calloc(cnt, sizeof(float));
  o->v = (float*)calloc(cnt, sizeof(float));
  o->e_srv = (float*)calloc(cnt, sizeof(float));
  o->e = (float*)calloc(cnt * (size_t)n, sizeof(float));
  o->c = (float*)calloc(keep_debug ? cnt * (size_t)n : (size_t)L, sizeof(float));
  o->u = (float*)calloc(dbg, sizeof(float));
  o->a = (float*)calloc(dbg, sizeof(float));
  o->wbits = (uint64_t*)calloc((size_t)o->words * (size_t)n, sizeof(uint64_t));
  o->sbits = (uint64_t*)calloc((size_t)o->words, sizeof(uint64_t));
  o->wscale = (float*)calloc((size_t)n * (size_t)o->nch, sizeof(float));
  o->sscale = (float*)calloc((size_t)o->nch, sizeof(float));
  o->vals = (float*)calloc((size_t)n, sizeof(float));
  if (!o->x || !o->m || !o->v || !o->e_srv || !o->e || !o->c || !o->u || !o->a || !o->wbits ||
      !o->sbits || !o->wscale || !o->sscale || !o->vals) {
    ob_oracle_destroy(o);
    return NULL;
  }
  return o;
}

void ob_oracle_destroy(ob_oracle* o) {
  if (!o) return;
  free(o->x);
  free(o->m);
  free(o->v);
  free(o->e_srv);
  free(o->e);
  free(o->c);
  free(o->u);
  free(o->a);
  free(o->wbits);
  free(o->sbits);
  free(o->wscale);
  free(o->sscale);
  free(o->vals);
  free(o->mloc);
  free(o->aloc);
  free(o->xloc);
  free(o);
}

/* Full-precision warm-up step: the workers' gradients are averaged exactly
 * as the server averages in the compression phase, then one step of Adam with
 * bias correction updates m, v and x ("Adam: A Method for Stochastic
 * Optimization", its Algorithm 1; epsilon outside the square root). */
void ob_oracle_warmup_step(ob_oracle* o, const void* const* grads, int32_t gdtype, float lr) {
  o->t += 1;
  double p1 = 1.0, p2 = 1.0;
  for (int64_t i = 0; i < o->t; ++i) {
    p1 = p1 * (double)o->beta1;
    p2 = p2 * (double)o->beta2;
  }
  const float bc1 = (float)(1.0 - p1);
  const float bc2 = (float)(1.0 - p2);
  const float ob1 = 1.0f - o->beta1;
  const float ob2 = 1.0f - o->beta2;
  for (int64_t k = 0; k < o->cnt; ++k) {
    for (int32_t w = 0; w < o->n; ++w) o->vals[w] = grad_at(grads[w], gdtype, k);
    float gbar = ob_oracle_pairwise_mean(o->vals, o->n);
    o->m[k] = (o->beta1 * o->m[k]) + (ob1 * gbar);
    o->v[k] = (o->beta2 * o->v[k]) + (ob2 * (gbar * gbar));
    float mh = o->m[k] / bc1;
    float vh = o->v[k] / bc2;
    o->x[k] = o->x[k] - lr * (mh / (sqrtf(vh) + o->eps));
  }
}

/* Worker w, held chunk jj: compensated values c[0..L) (already formed) ->
 * per-chunk scale, sign bits, new error e = c - (bit ? s : -s). */
static void worker_compress_chunk(ob_oracle* o, int32_t w, int32_t jj, const float* c,
                                  uint64_t* bits, float* e) {
  const int64_t L = o->L;
  const int64_t base = (int64_t)jj * L;
  float s = ob_oracle_chunk_scale(ob_oracle_chunk_sumsq(c, L), L);
  o->wscale[(size_t)w * (size_t)o->nch + jj] = s;
  for (int64_t q = 0; q < L; ++q) {
    int64_t k = base + q;
    int bit = c[q] >= 0.0f;
    set_bit(bits, k, bit);
    e[k] = c[q] - (bit ? s : -s);
  }
}

/* Server j (one per held chunk): average of the workers' decompressed
 * chunks, plus its own error; scale, sign bits, new error.  Every worker
 * then decompresses the server's chunk into m and updates x with the frozen
 * v by `step` (the step's learning rate). */
static void server_round(ob_oracle* o, float step) {
  const int32_t n = o->n;
  const int64_t L = o->L;
  memset(o->sbits, 0, sizeof(uint64_t) * (size_t)o->words);
  for (int32_t jj = 0; jj < o->nch; ++jj) {
    int64_t base = (int64_t)jj * L;
    float* a = o->keep_debug ? o->a + base : o->a;
    float* u = o->keep_debug ? o->u + base : o->u;
    for (int64_t q = 0; q < L; ++q) {
      int64_t k = base + q;
      for (int32_t w = 0; w < n; ++w) {
        float sw = o->wscale[(size_t)w * (size_t)o->nch + jj];
        o->vals[w] = get_bit(o->wbits + (size_t)w * (size_t)o->words, k) ? sw : -sw;
      }
      a[q] = ob_oracle_pairwise_mean(o->vals, n);
      u[q] = a[q] + o->e_srv[k];
    }
    float s = ob_oracle_chunk_scale(ob_oracle_chunk_sumsq(u, L), L);
    o->sscale[jj] = s;
    for (int64_t q = 0; q < L; ++q) {
      int64_t k = base + q;
      int bit = u[q] >= 0.0f;
      set_bit(o->sbits, k, bit);
      float t = bit ? s : -s;
      o->e_srv[k] = u[q] - t;
      o->m[k] = t;
      o->x[k] = o->x[k] - step * (o->m[k] / (sqrtf(o->v[k]) + o->eps));
    }
  }
}

/* Compression-phase step. */
void ob_oracle_compressed_step(ob_oracle* o, const void* const* grads, int32_t gdtype, float lr) {
  o->t += 1;
  const int32_t n = o->n;
  const int64_t L = o->L;
  const int64_t cnt = o->cnt;
  const float ob1 = 1.0f - o->beta1;

  /* Worker i: momentum from the shared m and its own gradient, plus its error
   * (error compensation); then per chunk: scale, sign bits, new error. */
  memset(o->wbits, 0, sizeof(uint64_t) * (size_t)o->words * (size_t)n);
  for (int32_t w = 0; w < n; ++w) {
    float* e = o->e + (size_t)w * (size_t)cnt;
    uint64_t* bits = o->wbits + (size_t)w * (size_t)o->words;
    for (int32_t jj = 0; jj < o->nch; ++jj) {
      int64_t base = (int64_t)jj * L;
      float* c = o->keep_debug ? o->c + (size_t)w * (size_t)cnt + base : o->c;
      for (int64_t q = 0; q < L; ++q) {
        int64_t k = base + q;
        float g = grad_at(grads[w], gdtype, k);
        c[q] = ((o->beta1 * o->m[k]) + (ob1 * g)) + e[k];
      }
      worker_compress_chunk(o, w, jj, c, bits, e);
    }
  }

  /* Server j (one per chunk): average of the workers' decompressed chunks,
   * plus its own error; scale, sign bits, new error.  Every worker then
   * decompresses the server's chunk into m and updates x with the frozen v. */
  server_round(o, lr);
}

void* ob_oracle_field(ob_oracle* o, int32_t field, int32_t worker, int64_t* count) {
  if (worker < 0 || worker >= o->n) worker = 0;
  size_t w = (size_t)worker;
  int64_t cnt = o->cnt;
  void* p = NULL;
  int64_t c = 0;
  switch (field) {
    case OBO_X: p = o->x; c = cnt; break;
    case OBO_M: p = o->m; c = cnt; break;
    case OBO_V: p = o->v; c = cnt; break;
    case OBO_E_WORKER: p = o->e + w * (size_t)cnt; c = cnt; break;
    case OBO_E_SERVER: p = o->e_srv; c = cnt; break;
    case OBO_C_WORKER:
      if (o->keep_debug) { p = o->c + w * (size_t)cnt; c = cnt; }
      break;
    case OBO_U_SERVER:
      if (o->keep_debug) { p = o->u; c = cnt; }
      break;
    case OBO_A_SERVER:
      if (o->keep_debug) { p = o->a; c = cnt; }
      break;
    case OBO_BITS_WORKER: p = o->wbits + w * (size_t)o->words; c = o->words; break;
    case OBO_BITS_SERVER: p = o->sbits; c = o->words; break;
    case OBO_SCALE_WORKER: p = o->wscale + w * (size_t)o->nch; c = o->nch; break;
    case OBO_SCALE_SERVER: p = o->sscale; c = o->nch; break;
    case OBO_M_LOCAL:
      if (o->mloc) { p = o->mloc + w * (size_t)cnt; c = cnt; }
      break;
    case OBO_A_LOCAL:
      if (o->aloc) { p = o->aloc + w * (size_t)cnt; c = cnt; }
      break;
    case OBO_X_LOCAL:
      if (o->xloc) {
        ob_oracle_zo_local_model(o, (int32_t)w, o->xloc);
        p = o->xloc;
        c = cnt;
      }
      break;
    default: break;
  }
  if (count) *count = c;
  return p;
}

int64_t ob_oracle_step(const ob_oracle* o) { return o->t; }
int64_t ob_oracle_held(const ob_oracle* o) { return o->cnt; }


/* ------------------------------------------------------------- 0/1 Adam --
 * "Maximizing Communication Efficiency for Large-scale Training via 0/1
 * Adam" (abstract): each Adam step is made linear by using stale estimates of
 * the optimizer state and the linear correlation between the momentum and
 * the model update; that linearity lets 1-bit compression and local steps
 * (rounds without communication) be combined.  The abstract fixes no
 * formula, so every step below is a reading (the design notes list them):
 *  - stale state: the variance v is refreshed only at the steps the caller
 *    flags, and only at a synchronizing step, by Adam's update on the
 *    full-precision worker average of that step's gradients; between
 *    refreshes it is frozen;
 *  - local steps: between synchronizations every worker runs momentum steps
 *    of its own, m_i = (b1*m_src) + ((1-b1)*g_i), with m_src the shared
 *    momentum at the first step of a local period and m_i afterwards;
 *  - linear correlation: with v frozen over the period, the worker's local
 *    model is x_sync - G*(a_i/(sqrtf(v)+eps)), where G is the sum of the
 *    period's step sizes and a_i the step-size-weighted mean of its momenta,
 *    kept as a_1 = m_1, a_k = a_{k-1} + (w_k*(m_k - a_{k-1})), w_k = g_k/G_k;
 *  - a synchronizing step sends a_i through the same 1-bit codec with error
 *    feedback as the compressed step (c_i = a_i + e_i, per-chunk scales,
 *    server average plus server error feedback); the decompressed server
 *    output becomes the shared momentum, x_sync -= G*(m/(sqrtf(v)+eps)), and
 *    the next step opens a new local period.
 * With a synchronization at every step and no refresh, each step equals
 * ob_oracle_compressed_step bit for bit (G = lr, a_i = m_i). */

static int zo_ready(ob_oracle* o) {
  if (o->mloc) return 1;
  o->mloc = (float*)calloc((size_t)o->cnt * (size_t)o->n, sizeof(float));
  o->aloc = (float*)calloc((size_t)o->cnt * (size_t)o->n, sizeof(float));
  o->xloc = (float*)calloc((size_t)o->cnt, sizeof(float));
  if (!o->mloc || !o->aloc || !o->xloc) abort();
  o->zgamma = 0.0f;
  o->zk = 0;
  return 1;
}

void ob_oracle_zo_step(ob_oracle* o, const void* const* grads, int32_t gdtype, float lr,
                       int32_t sync, int32_t refresh) {
  zo_ready(o);
  o->t += 1;
  const int32_t n = o->n;
  const int64_t L = o->L;
  const int64_t cnt = o->cnt;
  const float ob1 = 1.0f - o->beta1;
  const int first = o->zk == 0;

  /* the period's step sizes and this step's weight in the mean momentum */
  o->zgamma = first ? lr : o->zgamma + lr;
  const float wk = lr / o->zgamma;

  /* local momentum step of every worker, and its step-weighted mean */
  for (int32_t w = 0; w < n; ++w) {
    float* ml = o->mloc + (size_t)w * (size_t)cnt;
    float* al = o->aloc + (size_t)w * (size_t)cnt;
    for (int64_t k = 0; k < cnt; ++k) {
      float g = grad_at(grads[w], gdtype, k);
      float msrc = first ? o->m[k] : ml[k];
      float mi = (o->beta1 * msrc) + (ob1 * g);
      ml[k] = mi;
      al[k] = first ? mi : al[k] + (wk * (mi - al[k]));
    }
  }
  o->zk += 1;
  if (!sync) return;

  /* Synchronization.  Workers: compensated mean momentum, then the
   * compressed step's codec (per-chunk scale, sign bits, new error). */
  memset(o->wbits, 0, sizeof(uint64_t) * (size_t)o->words * (size_t)n);
  for (int32_t w = 0; w < n; ++w) {
    float* e = o->e + (size_t)w * (size_t)cnt;
    const float* al = o->aloc + (size_t)w * (size_t)cnt;
    uint64_t* bits = o->wbits + (size_t)w * (size_t)o->words;
    for (int32_t jj = 0; jj < o->nch; ++jj) {
      int64_t base = (int64_t)jj * L;
      float* c = o->keep_debug ? o->c + (size_t)w * (size_t)cnt + base : o->c;
      for (int64_t q = 0; q < L; ++q) c[q] = al[base + q] + e[base + q];
      worker_compress_chunk(o, w, jj, c, bits, e);
    }
  }

  /* Server: average, server error, re-compression; the decompressed output
   * is the shared momentum, and the shared model takes the period's summed
   * step sizes with the stale variance. */
  server_round(o, o->zgamma);

  /* Variance refresh (after the update, which used the stale one):
   * Adam's second-moment step on the full-precision average of this step's
   * gradients. */
  if (refresh) {
    const float ob2 = 1.0f - o->beta2;
    for (int64_t k = 0; k < cnt; ++k) {
      for (int32_t w = 0; w < n; ++w) o->vals[w] = grad_at(grads[w], gdtype, k);
      float gbar = ob_oracle_pairwise_mean(o->vals, n);
      o->v[k] = (o->beta2 * o->v[k]) + (ob2 * (gbar * gbar));
    }
  }
  o->zk = 0;
}

/* Worker w's local model: x_sync - G*(a_w/(sqrtf(v)+eps)) inside an open
 * local period, x_sync right after a synchronization. */
void ob_oracle_zo_local_model(ob_oracle* o, int32_t w, float* out) {
  const float* al = o->aloc ? o->aloc + (size_t)w * (size_t)o->cnt : NULL;
  for (int64_t k = 0; k < o->cnt; ++k) {
    if (o->zk == 0 || !al)
      out[k] = o->x[k];
    else
      out[k] = o->x[k] - o->zgamma * (al[k] / (sqrtf(o->v[k]) + o->eps));
  }
}

float ob_oracle_zo_gamma(const ob_oracle* o) { return o->zgamma; }
int32_t ob_oracle_zo_open(const ob_oracle* o) { return o->zk; }
