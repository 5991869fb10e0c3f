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
 *             noise from Philox4x64-10 keyed by (seed, t) (see oracle_gumbel);
 *             int8 rows use the scaled logits raw_v * s_r.
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
/* Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011): ten rounds of two 64 x 64 -> 128-bit products
 * of counter words with fixed multipliers, the high halves mixed with the other
 * counter words and the key, the key bumped by fixed Weyl constants between
 * rounds.  Counter and key are the whole state: output = f(counter, key). */
void oracle_philox4x64(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    unsigned __int128 p0 = (unsigned __int128)M0 * x0;
    unsigned __int128 p1 = (unsigned __int128)M1 * x2;
    uint64_t y0 = (uint64_t)(p1 >> 64) ^ x1 ^ k0, y1 = (uint64_t)p1;
    uint64_t y2 = (uint64_t)(p0 >> 64) ^ x3 ^ k1, y3 = (uint64_t)p0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Gumbel noise of token v for the draw keyed by (seed, position) ("12
 * Exactness", section 12.5: the token at index t is the argmax of
 * log p_t + G_t, G_t Gumbel noise from a generator seeded by (seed, t)).
 * Word (v >> 5) & 3 of Philox4x64-10 at counter (32 (v >> 7) + (v & 31), 0, 0, 0)
 * under key (seed, position); its top 23 bits u give U = (2u + 1) 2^-24 in
 * (0, 1); G = -ln(-ln U). */
double oracle_gumbel(uint64_t seed, int64_t position, int64_t v) {
  const uint64_t ctr[4] = {32 * (uint64_t)(v >> 7) + (uint64_t)(v & 31), 0, 0, 0};
  const uint64_t key[2] = {seed, (uint64_t)position};
  uint64_t out[4];
  oracle_philox4x64(ctr, key, out);
  const uint64_t u = out[(v >> 5) & 3] >> 41;
  const double U = (double)(2 * u + 1) * 0x1p-24;
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
