/*
 * oracle.c - plain, slow CPU reference of the batch-invariant LM head.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT.  Only tests/, __graft_entry__.smoke() and
 * bench.py's cpu_baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and neither uses the other.
 *
 * Every result is the plain definition, computed in float64 (bf16 inputs) or
 * exactly in int64 (int8 inputs):
 *
 *  logits     z[r][v] = sum_{k=0..H-1} x[r][k] * w[v][k], k ascending, one
 *             sequential accumulator.  A product of two bf16 values has at most
 *             16 significant bits, so every product is exact in float64 and the
 *             only rounding is the float64 running sum.
 *             ("Greedy Decoding Has a Precision Clause", section "Correct the
 *             vulnerable token decisions": the final output projection
 *             recomputed at higher precision; "Eliminating Nondeterminism in
 *             LLM Inference with Integer-Only Arithmetic", section "DetLLM":
 *             int8 x int8 -> int32 logits, exact in any order.)
 *  greedy     one scan v = 0..V-1 with strict comparisons, so the top-1 is the
 *             lowest id among the maxima and the top-2 the lowest id among the
 *             rest (an exactly tied maximum counts as "the rest"); the margin
 *             is z(1) - z(2).  (Precision Clause, "Token-ranking margins": the
 *             top-two logit margin; Integer-Only Arithmetic, "DetLLM": argmax
 *             breaks ties toward the lowest token id.)
 *  log-prob   m = max_v z, S = sum_v exp(z_v - m) (v ascending), then
 *             log p(t) = z_t - m - ln S; NaN when t is not in [0, V).
 *             ("Inference and Decoding", section 3, temperature softmax at
 *             tau = 1; "batch-logprob-gap": log probability of a given token.)
 *  int8 mode  top-2 and margin on the exact int64 logits, then the per-row
 *             positive scale s_r: value = float32((double)z * (double)s_r),
 *             one rounding of a product that is exact in float64 (|z| < 2^31,
 *             s_r has 24 significant bits).  Log-prob of the scaled logits
 *             with the differences taken exactly: S = sum exp(s_r (z_v - zmax)),
 *             log p(t) = s_r (z_t - zmax) - ln S.
 *
 *  sampling   seeded Gumbel-max: token = argmax_v z_v / T + G(seed, t, v), the
 *             noise from Philox4x32-10 keyed by (seed, t) (see oracle_gumbel);
 *             int8 rows use the scaled logits raw_v * s_r.
 *
 *  integer    the all-integer front and back of the int8 head, an algorithm
 *  front and  of our own stated in full at "integer front and back" below:
 *  back       per-token int8 quantisation with a dyadic step M 2^E, and a
 *             log-softmax in fixed point (Q.24 nats, exp values in Q.30) from
 *             exact integer logits, with one rounding rule (half up).
 *             ("Integer-Only Arithmetic", section "DetLLM": dyadic scales
 *             m / 2^k with one fixed rounding rule, shift-based integer
 *             exp and softmax, per-token activation quantisation.)
 *
 * Threads only split independent rows or independent vocab entries; the order
 * of every per-element sum is the one stated above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------ helpers */
static double bf16_value(uint16_t u) {
  uint32_t b = (uint32_t)u << 16;
  float f;
  memcpy(&f, &b, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 value (ties to even), returned as double.
 * bf16: 8 significant bits, exponent range of float32. */
double oracle_round_bf16(double z) {
  if (z == 0.0 || !isfinite(z)) return z;
  int e;
  double m = frexp(z, &e);            /* z = m * 2^e, 0.5 <= |m| < 1 */
  int p = 8;                          /* significant bits kept */
  if (e - 1 < -126) p -= (-126 - (e - 1));   /* subnormal bf16 */
  double q = nearbyint(ldexp(m, p));  /* default rounding mode: nearest-even */
  double r = ldexp(q, e - p);
  const double bf16_max = ldexp(255.0, 120);  /* (2 - 2^-7) * 2^127 */
  if (fabs(r) > bf16_max) r = copysign(INFINITY, z);
  return r;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/* A minimal parallel-for: threads pull task indices from a shared counter. */
typedef void (*task_fn)(void *ctx, int64_t task);
typedef struct {
  task_fn fn;
  void *ctx;
  int64_t ntasks;
  int64_t next;
  pthread_mutex_t mu;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t t = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (t >= p->ntasks) break;
    p->fn(p->ctx, t);
  }
  return NULL;
}

static void parallel_for(int nthreads, int64_t ntasks, task_fn fn, void *ctx) {
  if (ntasks <= 0) return;
  if (nthreads > ntasks) nthreads = (int)ntasks;
  pool_t p = {fn, ctx, ntasks, 0, PTHREAD_MUTEX_INITIALIZER};
  if (nthreads <= 1) {
    for (int64_t t = 0; t < ntasks; ++t) fn(ctx, t);
    return;
  }
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, pool_worker, &p) == 0) ++started;
  if (started == 0) pool_worker(&p);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------- logits */
enum { MODE_BF16 = 0, MODE_I8 = 1 };
#define VBLOCK 512

typedef struct {
  int mode;
  const void *x, *w;
  int64_t H, V, r0, nrows, nvb;
  void *z;  /* [nrows][V] double or int64 */
} logit_job;

static void logit_task(void *ctx, int64_t t) {
  const logit_job *j = (const logit_job *)ctx;
  int64_t rr = t / j->nvb, vb = t % j->nvb;
  int64_t r = j->r0 + rr, H = j->H, V = j->V;
  int64_t v0 = vb * VBLOCK, v1 = v0 + VBLOCK < V ? v0 + VBLOCK : V;
  if (j->mode == MODE_BF16) {
    const uint16_t *x = (const uint16_t *)j->x + r * H;
    const uint16_t *w = (const uint16_t *)j->w;
    double *z = (double *)j->z + rr * V;
    for (int64_t v = v0; v < v1; ++v) {
      const uint16_t *wv = w + v * H;
      double acc = 0.0;
      for (int64_t k = 0; k < H; ++k) acc += bf16_value(x[k]) * bf16_value(wv[k]);
      z[v] = acc;
    }
  } else {
    const int8_t *x = (const int8_t *)j->x + r * H;
    const int8_t *w = (const int8_t *)j->w;
    int64_t *z = (int64_t *)j->z + rr * V;
    for (int64_t v = v0; v < v1; ++v) {
      const int8_t *wv = w + v * H;
      int64_t acc = 0;
      for (int64_t k = 0; k < H; ++k) acc += (int64_t)x[k] * (int64_t)wv[k];
      z[v] = acc;
    }
  }
}

/* logits of rows [r0, r0+nrows) into z ([nrows][V]) */
static void logits_rows(int mode, const void *x, const void *w, int64_t H, int64_t V,
                        int64_t r0, int64_t nrows, void *z, int nthreads) {
  logit_job j = {mode, x, w, H, V, r0, nrows, (V + VBLOCK - 1) / VBLOCK, z};
  parallel_for(nthreads, nrows * j.nvb, logit_task, &j);
}

static int bad_shape(int64_t B, int64_t H, int64_t V) { return B < 0 || H < 1 || V < 1; }

int oracle_logits_bf16(const uint16_t *x, const uint16_t *w, int64_t B, int64_t H,
                       int64_t V, double *z, int nthreads) {
  if (bad_shape(B, H, V)) return 1;
  logits_rows(MODE_BF16, x, w, H, V, 0, B, z, resolve_threads(nthreads));
  return 0;
}

int oracle_logits_i8(const int8_t *x, const int8_t *w, int64_t B, int64_t H, int64_t V,
                     int64_t *z, int nthreads) {
  if (bad_shape(B, H, V)) return 1;
  logits_rows(MODE_I8, x, w, H, V, 0, B, z, resolve_threads(nthreads));
  return 0;
}

/* ------------------------------------------------- per-row definitions */
/* greedy top-2 of float64 logits (strict comparisons, lowest id wins ties) */
void oracle_top2_f64(const double *z, int64_t V, int32_t ids[2], double vals[2]) {
  double b1 = -INFINITY, b2 = -INFINITY;
  int64_t i1 = -1, i2 = -1;
  for (int64_t v = 0; v < V; ++v) {
    double t = z[v];
    if (i1 < 0 || t > b1) {
      b2 = b1; i2 = i1;
      b1 = t; i1 = v;
    } else if (i2 < 0 || t > b2) {
      b2 = t; i2 = v;
    }
  }
  ids[0] = (int32_t)i1; ids[1] = (int32_t)i2;
  vals[0] = b1; vals[1] = b2;
}

void oracle_top2_i64(const int64_t *z, int64_t V, int32_t ids[2], int64_t vals[2]) {
  int64_t b1 = 0, b2 = 0, i1 = -1, i2 = -1;
  for (int64_t v = 0; v < V; ++v) {
    int64_t t = z[v];
    if (i1 < 0 || t > b1) {
      b2 = b1; i2 = i1;
      b1 = t; i1 = v;
    } else if (i2 < 0 || t > b2) {
      b2 = t; i2 = v;
    }
  }
  ids[0] = (int32_t)i1; ids[1] = (int32_t)i2;
  vals[0] = b1; vals[1] = b2;
}

/* log-softmax of one float64 logit row: out[v] = z[v] - m - ln(sum exp(z - m)) */
void oracle_logsoftmax_f64(const double *z, int64_t V, double *out) {
  double m = -INFINITY;
  for (int64_t v = 0; v < V; ++v) if (z[v] > m) m = z[v];
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) s += exp(z[v] - m);
  double lse = m + log(s);
  for (int64_t v = 0; v < V; ++v) out[v] = z[v] - lse;
}

static double logprob_f64_row(const double *z, int64_t V, int64_t t) {
  if (t < 0 || t >= V) return NAN;
  double m = -INFINITY;
  for (int64_t v = 0; v < V; ++v) if (z[v] > m) m = z[v];
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) s += exp(z[v] - m);
  return z[t] - (m + log(s));
}

/* log p(t) of the scaled int logits s * z, differences taken exactly in int64 */
double oracle_logprob_i64_row(const int64_t *z, int64_t V, double scale, int64_t t) {
  if (t < 0 || t >= V || !(scale > 0.0) || !isfinite(scale)) return NAN;
  int64_t zmax = z[0];
  for (int64_t v = 1; v < V; ++v) if (z[v] > zmax) zmax = z[v];
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) s += exp(scale * (double)(z[v] - zmax));
  return scale * (double)(z[t] - zmax) - log(s);
}

/* ------------------------------------------- seeded Gumbel-max sampling */
/* Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit products
 * of counter words 0 and 2 with fixed multipliers; the new counter is (high
 * half of the second product ^ word 1 ^ key 0, its low half, high half of the
 * first product ^ word 3 ^ key 1, its low half); the key is bumped by fixed
 * Weyl constants between rounds.  Counter and key are the whole state:
 * output = f(counter, key). */
void oracle_philox4x32(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    uint64_t p0 = (uint64_t)M0 * x0;
    uint64_t p1 = (uint64_t)M1 * x2;
    uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0, y1 = (uint32_t)p1;
    uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1, y3 = (uint32_t)p0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Gumbel noise of token v for the draw keyed by (seed, position) ("12
 * Exactness", section 12.5: each token's log-probability plus Gumbel noise
 * from a generator keyed by the seed and the position; the largest sum is the
 * draw).
 * Word (v >> 5) & 3 of Philox4x32-10 at counter (32 (v >> 7) + (v & 31), 0,
 * position mod 2^32, position div 2^32) under key (seed mod 2^32, seed div
 * 2^32); its top 23 bits u give U = (2u + 1) 2^-24 in (0, 1); G = -ln(-ln U). */
double oracle_gumbel(uint64_t seed, int64_t position, int64_t v) {
  const uint64_t pos = (uint64_t)position;
  const uint32_t ctr[4] = {(uint32_t)(32 * (v >> 7) + (v & 31)), 0, (uint32_t)pos,
                           (uint32_t)(pos >> 32)};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32(ctr, key, out);
  const uint32_t u = out[(v >> 5) & 3] >> 9;
  const double U = (double)(2 * (uint64_t)u + 1) * 0x1p-24;
  return -log(-log(U));
}

/* ------------------------------------------------------- row pipelines */
/* rows are processed in chunks so the logits buffer stays near 256 MB */
static int64_t chunk_rows(int64_t B, int64_t V) {
  int64_t c = ((int64_t)256 << 20) / (V * 8);
  if (c < 1) c = 1;
  return c < B ? c : B;
}

typedef struct {
  int mode, round_bf16;
  int64_t V, r0;
  const void *z;
  const float *scale;
  const int32_t *target;
  int32_t *ids;
  double *vals_d, *margin_d, *logp;
  int64_t *raw;
  float *vals_f, *margin_f;
  double temperature;       /* sampling */
  const uint64_t *seed;
  const int64_t *position;
  int32_t *token;
  double *value, *gap;
} scan_job;

static float scaled_f32(int64_t z, float s) {
  if (!(s > 0.0f) || !isfinite(s)) return NAN;
  return (float)((double)z * (double)s);
}

static void greedy_task(void *ctx, int64_t rr) {
  const scan_job *j = (const scan_job *)ctx;
  int64_t r = j->r0 + rr, V = j->V;
  if (j->mode == MODE_BF16) {
    const double *z = (const double *)j->z + rr * V;
    double *tmp = NULL;
    if (j->round_bf16) {
      tmp = (double *)malloc(sizeof(double) * (size_t)V);
      for (int64_t v = 0; v < V; ++v) tmp[v] = oracle_round_bf16(z[v]);
      z = tmp;
    }
    int32_t ids[2];
    double vals[2];
    oracle_top2_f64(z, V, ids, vals);
    j->ids[2 * r] = ids[0]; j->ids[2 * r + 1] = ids[1];
    j->vals_d[2 * r] = vals[0]; j->vals_d[2 * r + 1] = vals[1];
    j->margin_d[r] = vals[0] - vals[1];
    free(tmp);
  } else {
    const int64_t *z = (const int64_t *)j->z + rr * V;
    int32_t ids[2];
    int64_t vals[2];
    oracle_top2_i64(z, V, ids, vals);
    float s = j->scale ? j->scale[r] : 1.0f;
    j->ids[2 * r] = ids[0]; j->ids[2 * r + 1] = ids[1];
    j->raw[2 * r] = vals[0]; j->raw[2 * r + 1] = vals[1];
    j->vals_f[2 * r] = scaled_f32(vals[0], s);
    j->vals_f[2 * r + 1] = scaled_f32(vals[1], s);
    j->margin_f[r] = scaled_f32(vals[0] - vals[1], s);
  }
}

static void logprob_task(void *ctx, int64_t rr) {
  const scan_job *j = (const scan_job *)ctx;
  int64_t r = j->r0 + rr, V = j->V;
  if (j->mode == MODE_BF16)
    j->logp[r] = logprob_f64_row((const double *)j->z + rr * V, V, j->target[r]);
  else
    j->logp[r] = oracle_logprob_i64_row((const int64_t *)j->z + rr * V, V,
                                        j->scale ? (double)j->scale[r] : 1.0, j->target[r]);
}

/* y_v = z_v / T + G(seed, position, v) for every token, then the top two with
 * strict comparisons (the lowest id wins a tie).  int8: z_v = raw_v * scale. */
static void sample_task(void *ctx, int64_t rr) {
  const scan_job *j = (const scan_job *)ctx;
  int64_t r = j->r0 + rr, V = j->V;
  double s = 1.0;
  if (j->mode == MODE_I8 && j->scale) {
    s = (double)j->scale[r];
    if (!(s > 0.0) || !isfinite(s)) {
      j->token[r] = -1; j->value[r] = NAN; j->gap[r] = NAN;
      return;
    }
  }
  double b1 = -INFINITY, b2 = -INFINITY;
  int32_t i1 = -1;
  for (int64_t v = 0; v < V; ++v) {
    double z = j->mode == MODE_BF16 ? ((const double *)j->z)[rr * V + v]
                                    : (double)((const int64_t *)j->z)[rr * V + v] * s;
    double y = z / j->temperature + oracle_gumbel(j->seed[r], j->position[r], v);
    if (y > b1) { b2 = b1; b1 = y; i1 = (int32_t)v; }
    else if (y > b2) { b2 = y; }
  }
  j->token[r] = i1; j->value[r] = b1; j->gap[r] = b1 - b2;
}

static int run_rows(scan_job *job, const void *x, const void *w, int64_t B, int64_t H,
                    task_fn fn, int nthreads) {
  int64_t V = job->V, c = chunk_rows(B, V);
  void *z = malloc((size_t)(c * V * 8));
  if (!z) return 2;
  nthreads = resolve_threads(nthreads);
  for (int64_t r0 = 0; r0 < B; r0 += c) {
    int64_t n = (B - r0 < c) ? B - r0 : c;
    logits_rows(job->mode, x, w, H, V, r0, n, z, nthreads);
    job->r0 = r0;
    job->z = z;
    parallel_for(nthreads, n, fn, job);
  }
  free(z);
  return 0;
}

int oracle_greedy_bf16(const uint16_t *x, const uint16_t *w, int64_t B, int64_t H, int64_t V,
                       int round_bf16, int32_t *ids, double *vals, double *margin,
                       int nthreads) {
  if (bad_shape(B, H, V) || V < 2) return 1;
  scan_job j;
  memset(&j, 0, sizeof j);
  j.mode = MODE_BF16; j.round_bf16 = round_bf16; j.V = V;
  j.ids = ids; j.vals_d = vals; j.margin_d = margin;
  return run_rows(&j, x, w, B, H, greedy_task, nthreads);
}

int oracle_greedy_i8(const int8_t *x, const int8_t *w, int64_t B, int64_t H, int64_t V,
                     const float *scale, int32_t *ids, int64_t *raw, float *vals,
                     float *margin, int nthreads) {
  if (bad_shape(B, H, V) || V < 2) return 1;
  scan_job j;
  memset(&j, 0, sizeof j);
  j.mode = MODE_I8; j.V = V; j.scale = scale;
  j.ids = ids; j.raw = raw; j.vals_f = vals; j.margin_f = margin;
  return run_rows(&j, x, w, B, H, greedy_task, nthreads);
}

int oracle_logprob_bf16(const uint16_t *x, const uint16_t *w, int64_t B, int64_t H, int64_t V,
                        const int32_t *target, double *logp, int nthreads) {
  if (bad_shape(B, H, V)) return 1;
  scan_job j;
  memset(&j, 0, sizeof j);
  j.mode = MODE_BF16; j.V = V; j.target = target; j.logp = logp;
  return run_rows(&j, x, w, B, H, logprob_task, nthreads);
}

int oracle_logprob_i8(const int8_t *x, const int8_t *w, int64_t B, int64_t H, int64_t V,
                      const float *scale, const int32_t *target, double *logp, int nthreads) {
  if (bad_shape(B, H, V)) return 1;
  scan_job j;
  memset(&j, 0, sizeof j);
  j.mode = MODE_I8; j.V = V; j.scale = scale; j.target = target; j.logp = logp;
  return run_rows(&j, x, w, B, H, logprob_task, nthreads);
}

int oracle_sample_bf16(const uint16_t *x, const uint16_t *w, int64_t B, int64_t H, int64_t V,
                       double temperature, const uint64_t *seed, const int64_t *position,
                       int32_t *token, double *value, double *gap, int nthreads) {
  if (bad_shape(B, H, V) || V < 2 || !(temperature > 0.0)) return 1;
  scan_job j;
  memset(&j, 0, sizeof j);
  j.mode = MODE_BF16; j.V = V; j.temperature = temperature; j.seed = seed; j.position = position;
  j.token = token; j.value = value; j.gap = gap;
  return run_rows(&j, x, w, B, H, sample_task, nthreads);
}

int oracle_sample_i8(const int8_t *x, const int8_t *w, int64_t B, int64_t H, int64_t V,
                     const float *scale, double temperature, const uint64_t *seed,
                     const int64_t *position, int32_t *token, double *value, double *gap,
                     int nthreads) {
  if (bad_shape(B, H, V) || V < 2 || !(temperature > 0.0)) return 1;
  scan_job j;
  memset(&j, 0, sizeof j);
  j.mode = MODE_I8; j.V = V; j.scale = scale; j.temperature = temperature; j.seed = seed;
  j.position = position; j.token = token; j.value = value; j.gap = gap;
  return run_rows(&j, x, w, B, H, sample_task, nthreads);
}

int oracle_threads(int nthreads) { return resolve_threads(nthreads); }

/* ------------------------------------------------ integer front and back */
/* The pages name the ingredients (dyadic scales m / 2^k rescaled by an integer
 * multiply and a shift with one rounding rule; shift-based integer exp and
 * softmax; each token quantised from its own values) but print no algorithm.
 * This is ours, every step in integers:
 *
 *  rounding   every rescale rounds half up: rnd(p, s) = floor((p + 2^(s-1)) / 2^s)
 *             on a non-negative p; a rounded division is floor((2a + b) / 2b).
 *
 *  front      row x (int32) -> q (int8) and step D = M 2^E, 2^14 <= M < 2^15:
 *             a = max |x|; D is the least number with a 15-bit mantissa such
 *             that 127 D >= a (a zero row: q = 0, D = 1 = 2^14 2^-14);
 *             q = sign(x) round_half_away(|x| / D), so |q| <= 127 and the
 *             largest |x| maps to 127.
 *
 *  scale      a row's logit z = sum q w has the real value z * m / 2^k:
 *             m / 2^k = U * D with the tensor unit U = um 2^ue (the real value
 *             of one unit of x times one unit of w), the mantissa product
 *             um * M rounded to 31 bits; valid when 24 <= k <= 86.
 *
 *  exp        iexp(T) = e^(-T / 2^24) in Q.30 for T >= 0 in Q.24 nats:
 *             T = q L + r with L = round(ln 2 * 2^24), 0 <= r < L; e^(-r/2^24)
 *             by its Taylor series to degree 10 in Horner form with the
 *             coefficients C_n = round(2^30 / n!); then times 2^-q by rnd.
 *
 *  ln         iln(S) = ln(S / 2^30) in Q.30 for S >= 2^30: S = 2^l (1 + f),
 *             ln(1 + f) = 2 atanh(u), u = f / (2 + f) < 1/3, the odd series
 *             to u^25; plus (l - 30) round(ln 2 * 2^30).
 *
 *  softmax    blocks of 128 vocabulary columns (b = v / 128, fixed by V):
 *             m_b = max z over the block; S_b = sum iexp(T(m_b - z_v));
 *             z_max = max m_b; S = sum_b rnd(S_b * iexp(T(z_max - m_b)), 30);
 *             T(d) = rnd(d * m, k - 24); all sums exact, so in any order.
 *             log p(t) = -(T(z_max - z_t) + rnd(iln(S), 6)) in Q.24 (int64,
 *             at least -(2^63 - 1)); INT64_MIN when t is not in [0, V) or the
 *             scale is not valid.
 */
#define FIX_NATS 24   /* fractional bits of a value in nats */
#define FIX_EXP 30    /* fractional bits of an exp value and of ln inside iln */
#define EXP_DEGREE 10
#define ATANH_TERMS 12

static uint64_t rnd(uint64_t p, int s) {   /* p < 2^63 */
  if (s <= 0) return p;
  if (s >= 64) return 0;
  return (p + ((uint64_t)1 << (s - 1))) >> s;
}

static uint64_t rnd_div(uint64_t a, uint64_t b) { return (2 * a + b) / (2 * b); }

static int bit_length(uint64_t v) {
  int n = 0;
  while (v) { ++n; v >>= 1; }
  return n;
}

/* round(ln 2 * 2^frac): log(2.0) is within 1e-16 of ln 2 and the product is
 * more than 1e-4 away from a rounding boundary for frac = 24 and 30 */
static uint64_t ln2_fixed(int frac) { return (uint64_t)llround(log(2.0) * ldexp(1.0, frac)); }

static uint64_t factorial(int n) {
  uint64_t f = 1;
  for (int i = 2; i <= n; ++i) f *= (uint64_t)i;
  return f;
}

uint64_t oracle_iexp_q30(uint64_t T) {
  const uint64_t L = ln2_fixed(FIX_NATS);
  if (T >= 64 * L) return 0;  /* q >= 64: 2^-q of a Q.30 value rounds to 0 */
  const uint64_t q = T / L, r = T - q * L;
  uint64_t y = rnd_div((uint64_t)1 << FIX_EXP, factorial(EXP_DEGREE));
  for (int n = EXP_DEGREE - 1; n >= 0; --n) {
    const uint64_t c = rnd_div((uint64_t)1 << FIX_EXP, factorial(n));
    y = c - rnd(y * r, FIX_NATS);  /* y <= 2^30, r < 2^24; y stays positive */
  }
  return rnd(y, (int)q);
}

int64_t oracle_iln_q30(uint64_t S) {
  if (S < ((uint64_t)1 << FIX_EXP)) return INT64_MIN;
  int l = bit_length(S) - 1;                       /* 2^l <= S < 2^(l+1) */
  uint64_t mant = rnd(S, l - FIX_EXP);             /* in [2^30, 2^31] */
  if (mant == ((uint64_t)2 << FIX_EXP)) { mant = (uint64_t)1 << FIX_EXP; l += 1; }
  const uint64_t f = mant - ((uint64_t)1 << FIX_EXP);
  const uint64_t u = rnd_div(f << FIX_EXP, ((uint64_t)2 << FIX_EXP) + f);
  const uint64_t u2 = rnd(u * u, FIX_EXP);
  uint64_t t = u, acc = u;
  for (int j = 1; j <= ATANH_TERMS; ++j) {
    t = rnd(t * u2, FIX_EXP);
    acc += rnd_div(t, (uint64_t)(2 * j + 1));
  }
  return (int64_t)(l - FIX_EXP) * (int64_t)ln2_fixed(FIX_EXP) + 2 * (int64_t)acc;
}

/* logit scale m / 2^k of a row from the tensor unit um 2^ue and the row step
 * M 2^E; returns 0 (invalid) unless um, M > 0 and 24 <= k <= 86 */
int oracle_int_row_scale(int32_t um, int32_t ue, int32_t M, int32_t E, int64_t *m, int32_t *k) {
  if (um <= 0 || M <= 0) return 0;
  const uint64_t P = (uint64_t)um * (uint64_t)M;   /* < 2^62 */
  int sh = bit_length(P) - 31;
  uint64_t mm;
  if (sh > 0) {
    mm = rnd(P, sh);
    if (mm == ((uint64_t)1 << 31)) { mm = (uint64_t)1 << 30; sh += 1; }
  } else {
    mm = P << (-sh);
  }
  const int64_t kk = -((int64_t)sh + ue + E);       /* real = mm 2^(sh + ue + E) */
  if (kk < FIX_NATS || kk > FIX_NATS + 62) return 0;
  *m = (int64_t)mm;
  *k = (int32_t)kk;
  return 1;
}

void oracle_quantize_row(const int32_t *x, int64_t H, int8_t *q, int32_t *M, int32_t *E) {
  uint64_t a = 0;
  for (int64_t i = 0; i < H; ++i) {
    const uint64_t v = x[i] < 0 ? (uint64_t)(-(int64_t)x[i]) : (uint64_t)x[i];
    if (v > a) a = v;
  }
  if (a == 0) {
    for (int64_t i = 0; i < H; ++i) q[i] = 0;
    *M = 1 << 14; *E = -14;
    return;
  }
  /* e = floor(log2(a / 127)): the largest e with 127 2^e <= a */
  int e = 40;
  for (;; --e) {
    const int ok = e >= 0 ? ((uint64_t)127 << e) <= a : (uint64_t)127 <= (a << (-e));
    if (ok) break;
  }
  int ee = e - 14;                                  /* D = M 2^ee */
  uint64_t mm;
  if (ee <= 0) {
    mm = ((a << (-ee)) + 126) / 127;                /* ceil(a 2^-ee / 127) */
  } else {
    const uint64_t d = (uint64_t)127 << ee;
    mm = (a + d - 1) / d;
  }
  if (mm == ((uint64_t)1 << 15)) { mm = (uint64_t)1 << 14; ee += 1; }
  const uint64_t num_shift = ee < 0 ? (uint64_t)(-ee) : 0, D = mm << (ee > 0 ? ee : 0);
  for (int64_t i = 0; i < H; ++i) {
    const uint64_t v = x[i] < 0 ? (uint64_t)(-(int64_t)x[i]) : (uint64_t)x[i];
    const uint64_t n = v << num_shift;
    const int64_t r = (int64_t)((2 * n + D) / (2 * D));   /* round half away from zero */
    q[i] = (int8_t)(x[i] < 0 ? -r : r);
  }
  *M = (int32_t)mm;
  *E = (int32_t)ee;
}

int oracle_quantize_rows(const int32_t *x, int64_t B, int64_t H, int8_t *q, int32_t *M,
                         int32_t *E) {
  if (B < 0 || H < 1) return 1;
  for (int64_t r = 0; r < B; ++r) oracle_quantize_row(x + r * H, H, q + r * H, M + r, E + r);
  return 0;
}

/* one row of exact integer logits (|z| < 2^31) -> log p(t) in Q.24 */
int64_t oracle_logprob_int_row(const int64_t *z, int64_t V, int64_t m, int32_t k, int64_t t) {
  if (t < 0 || t >= V || m <= 0 || k < FIX_NATS || k > FIX_NATS + 62) return INT64_MIN;
  const int sh = k - FIX_NATS;
  const int64_t nb = (V + 127) / 128;
  int64_t zmax = INT64_MIN;
  for (int64_t v = 0; v < V; ++v) if (z[v] > zmax) zmax = z[v];
  uint64_t S = 0;
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t v0 = b * 128, v1 = v0 + 128 < V ? v0 + 128 : V;
    int64_t mb = INT64_MIN;
    for (int64_t v = v0; v < v1; ++v) if (z[v] > mb) mb = z[v];
    uint64_t Sb = 0;
    for (int64_t v = v0; v < v1; ++v)
      Sb += oracle_iexp_q30(rnd((uint64_t)(mb - z[v]) * (uint64_t)m, sh));
    const uint64_t R = oracle_iexp_q30(rnd((uint64_t)(zmax - mb) * (uint64_t)m, sh));
    /* rnd(Sb * R, 30) with Sb < 2^38: split Sb at bit 32 so both products fit */
    S += ((Sb >> 32) * R << 2) + rnd((Sb & 0xffffffffu) * R, FIX_EXP);
  }
  const uint64_t Tt = rnd((uint64_t)(zmax - z[t]) * (uint64_t)m, sh);
  const uint64_t L = rnd((uint64_t)oracle_iln_q30(S), FIX_EXP - FIX_NATS);
  const uint64_t nl = Tt + L;                  /* < 2^63 + 2^40: no wrap */
  return nl > (uint64_t)INT64_MAX ? -INT64_MAX : -(int64_t)nl;
}

typedef struct {
  int64_t V, r0;
  const int64_t *z;
  const int64_t *m;
  const int32_t *k, *target;
  int64_t *logp;
} int_job;

static void logprob_int_task(void *ctx, int64_t rr) {
  const int_job *j = (const int_job *)ctx;
  const int64_t r = j->r0 + rr;
  j->logp[r] = oracle_logprob_int_row(j->z + rr * j->V, j->V, j->m[r], j->k[r], j->target[r]);
}

/* x, w int8; per-row logit scale from the unit (um, ue) and the row steps
 * (M, E); log p(target) in Q.24 */
int oracle_logprob_int(const int8_t *x, const int8_t *w, int64_t B, int64_t H, int64_t V,
                       int32_t um, int32_t ue, const int32_t *M, const int32_t *E,
                       const int32_t *target, int64_t *logp, int nthreads) {
  if (bad_shape(B, H, V)) return 1;
  int64_t *m = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B ? B : 1));
  int32_t *k = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B ? B : 1));
  int64_t c = chunk_rows(B, V);
  int64_t *z = (int64_t *)malloc((size_t)(c * V * 8));
  if (!m || !k || !z) { free(m); free(k); free(z); return 2; }
  for (int64_t r = 0; r < B; ++r)
    if (!oracle_int_row_scale(um, ue, M[r], E[r], &m[r], &k[r])) { m[r] = 0; k[r] = 0; }
  nthreads = resolve_threads(nthreads);
  int_job j = {V, 0, z, m, k, target, logp};
  for (int64_t r0 = 0; r0 < B; r0 += c) {
    const int64_t n = (B - r0 < c) ? B - r0 : c;
    logits_rows(MODE_I8, x, w, H, V, r0, n, z, nthreads);
    j.r0 = r0;
    parallel_for(nthreads, n, logprob_int_task, &j);
  }
  free(m); free(k); free(z);
  return 0;
}

