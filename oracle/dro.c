/*
 * dro.c -- CPU oracle for batch-invariant MoE routing.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg load this library.  It is the plain
 * definition of the routing path, written step by step; nothing here is
 * blocked, fused or reordered.  See dro.h for the sources and readings.
 *
 * Compile with -ffp-contract=off and without fast-math: every fused
 * multiply-add below is an explicit fmaf(), every other operation is a single
 * IEEE fp32 operation rounded to nearest even.
 */
#define _GNU_SOURCE
#include "dro.h"

#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>
#include <limits.h>

/* ------------------------------------------------------------------ bits */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float bf16_widen(uint16_t b) { return u2f((uint32_t)b << 16); }

/* bf16 RNE.  Reading taken: the pages name bf16 values and "representable
 * bf16 steps" (vllm.cpp PR #2556, summary) without a rounding rule; round to
 * nearest, ties to even, as hardware conversions do, and every NaN becomes the
 * canonical quiet NaN 0x7FC0. */
uint16_t dro_bf16_rne(float v) {
  uint32_t u = f2u(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  uint32_t lower = u & 0xFFFFu;
  uint32_t upper = u >> 16;
  /* round half to even on the 16 discarded bits */
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* Sign-magnitude total order (vllm.cpp PR #2556, "Why a value tap could never
 * have said this": the margin is counted in bf16 ULPs under this order, and
 * ulps = 0 means the same bf16 value).  Reading: negative patterns map to the
 * negated magnitude, so -0 and +0 both map to 0. */
int32_t dro_bf16_ord(uint16_t b) {
  int32_t mag = (int32_t)(b & 0x7FFFu);
  return (b & 0x8000u) ? -mag : mag;
}

int32_t dro_ulps(uint16_t a, uint16_t b) { return dro_bf16_ord(a) - dro_bf16_ord(b); }

/* ------------------------------------------------------------------ exp */

/* Reading: the pages leave the softmax's exponential open (vllm.cpp PR #2556
 * only calls the denominator a device-order f32 reduction).  To make the
 * weights a defined function of the logits, the routing path uses its own
 * exponential for t <= 0:
 *   n = rint(t * log2(e))            (fp32 multiply, then round half even)
 *   r = t - n*ln2                    (two fmaf steps, ln2 split hi + lo)
 *   p = sum_{i=0..7} r^i / i!        (Horner with fmaf, fp32 coefficients)
 *   exp(t) = p * 2^n                 (one fp32 multiply by an exact power of 2)
 * with t < -87 giving +0 (so n >= -126 and 2^n is a normal float).  Its
 * accuracy against the true exponential is what the tests pin. */
static const float LOG2E_F = 0x1.715476p+0f;
static const float LN2_HI_F = 0x1.62e43p-1f;
static const float LN2_LO_F = -0x1.05c61p-29f;
static const float INV_FACT_F[8] = {
    0x1.0p+0f,       /* 1/0! */
    0x1.0p+0f,       /* 1/1! */
    0x1.0p-1f,       /* 1/2! */
    0x1.555556p-3f,  /* 1/3! */
    0x1.555556p-5f,  /* 1/4! */
    0x1.111112p-7f,  /* 1/5! */
    0x1.6c16c2p-10f, /* 1/6! */
    0x1.a01a02p-13f, /* 1/7! */
};

float dro_expf(float t) {
  if (!(t <= 0.0f)) return u2f(0x7FC00000u); /* t > 0 or NaN: outside the domain */
  if (t < -87.0f) return 0.0f;
  float n = rintf(t * LOG2E_F);
  float r = fmaf(-n, LN2_HI_F, t);
  r = fmaf(-n, LN2_LO_F, r);
  float p = INV_FACT_F[7];
  for (int i = 6; i >= 0; --i) p = fmaf(p, r, INV_FACT_F[i]);
  int ni = (int)n; /* in [-126, 0] */
  float scale = u2f((uint32_t)(ni + 127) << 23);
  return p * scale;
}

void dro_expf_array(const float *t, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = dro_expf(t[i]);
}

/* ------------------------------------------------------------------ tree */

/* The fixed pairwise tree ("The Illusion of Determinism...", section "The
 * anatomy of the missing numeric contract": the contract must fix the
 * associative grouping of the K reduction).  Reading: combine adjacent pairs
 * level by level, q_i = v_{2i} + v_{2i+1}; an odd last element moves up a
 * level unchanged; repeat until one value is left.  Works in place on v. */
static float pairwise_tree(float *v, int64_t n) {
  if (n <= 0) return 0.0f;
  while (n > 1) {
    int64_t half = n / 2;
    for (int64_t i = 0; i < half; ++i) v[i] = v[2 * i] + v[2 * i + 1];
    if (n & 1) v[half] = v[n - 1];
    n = half + (n & 1);
  }
  return v[0];
}

/* ------------------------------------------------------------------ dot */

static float x_at(const void *x, int x_is_bf16, int64_t K, int64_t m, int64_t kk) {
  if (x_is_bf16) return bf16_widen(((const uint16_t *)x)[m * K + kk]);
  return ((const float *)x)[m * K + kk];
}

/* Canonical dot of row m with column e of W (stride E): one fmaf chain from
 * +0 per K-block of `kblock` consecutive k in ascending order, then the tree
 * over the block partials.  ("Batch changed the model's mind", section "The
 * fix: m-invariant twins": a fixed reduction order per row, independent of
 * how many rows share the launch.)  `part` is scratch of ceil(K/kblock). */
static float canonical_dot(const void *x, int x_is_bf16, const float *W, int64_t K, int64_t E,
                           int64_t m, int64_t e, int64_t kblock, float *part) {
  int64_t nb = (K + kblock - 1) / kblock;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t k0 = b * kblock;
    int64_t k1 = k0 + kblock < K ? k0 + kblock : K;
    float p = 0.0f;
    for (int64_t kk = k0; kk < k1; ++kk) p = fmaf(x_at(x, x_is_bf16, K, m, kk), W[kk * E + e], p);
    part[b] = p;
  }
  return pairwise_tree(part, nb);
}

/* Positive-control dot: s contiguous slices of K (sizes as even as integer
 * division allows), each a sequential fmaf chain from +0, summed left to
 * right.  A library that picks s from M behaves like this. */
static float split_dot(const void *x, int x_is_bf16, const float *W, int64_t K, int64_t E,
                       int64_t m, int64_t e, int64_t s) {
  float total = 0.0f;
  for (int64_t j = 0; j < s; ++j) {
    int64_t k0 = K * j / s, k1 = K * (j + 1) / s;
    float p = 0.0f;
    for (int64_t kk = k0; kk < k1; ++kk) p = fmaf(x_at(x, x_is_bf16, K, m, kk), W[kk * E + e], p);
    total = (j == 0) ? p : total + p;
  }
  return total;
}

static int64_t split_factor(int64_t M) { return M <= 64 ? 1 : (M <= 74 ? 2 : 4); }

/* ------------------------------------------------------------------ select */

/* Ranking key order (vllm.cpp PR #2556, summary: at a tie the lowest index
 * wins).  Reading: larger value first; equal values (IEEE equality, so +0 and
 * -0 tie) by ascending index; NaN ranks below every number, NaNs among
 * themselves by ascending index. */
typedef struct {
  float v;
  int32_t i;
} ent_t;

static int rank_cmp(const void *pa, const void *pb) {
  const ent_t *a = (const ent_t *)pa, *b = (const ent_t *)pb;
  int an = isnan(a->v), bn = isnan(b->v);
  if (an != bn) return an ? 1 : -1;
  if (!an) {
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
  }
  return (a->i < b->i) ? -1 : (a->i > b->i ? 1 : 0);
}

/* One token: given its E logits (already canonical, fp32), apply the optional
 * bf16 rounding, rank, and fill ids / weights / margin. */
static void route_token(const float *logit_in, int64_t E, int32_t k, int logits_bf16,
                        uint32_t flags, float *l, ent_t *ent, float *u, int32_t *ids,
                        float *weights, float *sel_logits, dro_margin *margin) {
  for (int64_t e = 0; e < E; ++e) {
    float v = logit_in[e];
    /* vllm.cpp PR #2556, "Why a value tap...": the bf16 logits are what the
     * selection is a function of. */
    l[e] = logits_bf16 ? bf16_widen(dro_bf16_rne(v)) : v;
    if (sel_logits) sel_logits[e] = l[e];
  }
  for (int64_t e = 0; e < E; ++e) {
    ent[e].v = l[e];
    ent[e].i = (int32_t)e;
  }
  qsort(ent, (size_t)E, sizeof(ent_t), rank_cmp);
  for (int32_t j = 0; j < k; ++j) ids[j] = ent[j].i;

  if (margin) {
    float sel = ent[k - 1].v;
    float rej = (k < E) ? ent[k].v : -INFINITY;
    margin->sel_min = sel;
    margin->rej_max = rej;
    margin->sel_min_bf16 = dro_bf16_rne(sel);
    margin->rej_max_bf16 = dro_bf16_rne(rej);
    margin->ulps = (k < E) ? dro_ulps(margin->sel_min_bf16, margin->rej_max_bf16) : INT32_MAX;
  }

  if (weights) {
    /* Softmax over all E logits, gathered at the selected ids.  Reading: the
     * maximum is the top-ranked value; u_e = exp(l_e - max) with dro_expf; the
     * denominator is the pairwise tree over u_0..u_{E-1} in index order; each
     * weight is one IEEE division.  Optional renormalisation divides by the
     * left-to-right sum of the k weights in rank order. */
    float mx = ent[0].v;
    for (int64_t e = 0; e < E; ++e) u[e] = dro_expf(l[e] - mx);
    float *tmp = u + E;
    memcpy(tmp, u, (size_t)E * sizeof(float));
    float s = pairwise_tree(tmp, E);
    for (int32_t j = 0; j < k; ++j) weights[j] = u[ids[j]] / s;
    if (flags & 1u) {
      float r = weights[0];
      for (int32_t j = 1; j < k; ++j) r = r + weights[j];
      for (int32_t j = 0; j < k; ++j) weights[j] = weights[j] / r;
    }
  }
}

/* ------------------------------------------------------------------ threads */

int dro_default_threads(void) {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  return 1;
}

typedef struct job job_t;
typedef void (*row_fn)(job_t *, int64_t m, void *scratch);

struct job {
  row_fn fn;
  int64_t M;
  int64_t next; /* rows handed out in fixed contiguous chunks per thread */
  int nthreads;
  size_t scratch_bytes;
  /* route */
  const void *x;
  int x_is_bf16;
  const float *W;
  int64_t K, E;
  int32_t k;
  int64_t kblock;
  int logits_bf16;
  uint32_t flags;
  int split_mode;
  int32_t *ids;
  float *weights, *sel_logits, *logits_out;
  const float *logits_in;
  dro_margin *margins;
  /* gate / gemm */
  const void *w;
  int w_is_bf16;
  float *dot, *gate;
  const uint16_t *xb, *Wb;
  int64_t N;
  float *out;
  /* grouped gemm */
  const int32_t *src_rows, *expert_of;
};

typedef struct {
  job_t *job;
  int t;
} targ_t;

static void *thread_main(void *p) {
  targ_t *a = (targ_t *)p;
  job_t *j = a->job;
  int64_t per = (j->M + j->nthreads - 1) / j->nthreads;
  int64_t m0 = per * a->t, m1 = m0 + per < j->M ? m0 + per : j->M;
  void *scratch = j->scratch_bytes ? malloc(j->scratch_bytes) : NULL;
  for (int64_t m = m0; m < m1; ++m) j->fn(j, m, scratch);
  free(scratch);
  return NULL;
}

static void run_rows(job_t *j, int nthreads) {
  if (nthreads <= 0) nthreads = dro_default_threads();
  if (j->M <= 0) return;
  if (nthreads > j->M) nthreads = (int)j->M;
  j->nthreads = nthreads;
  pthread_t th[1024];
  targ_t args[1024];
  if (nthreads > 1024) nthreads = j->nthreads = 1024;
  for (int t = 0; t < nthreads; ++t) {
    args[t].job = j;
    args[t].t = t;
    if (t > 0) pthread_create(&th[t], NULL, thread_main, &args[t]);
  }
  thread_main(&args[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ logits */

static void logits_row(job_t *j, int64_t m, void *scratch) {
  float *part = (float *)scratch;
  for (int64_t e = 0; e < j->E; ++e)
    j->logits_out[m * j->E + e] = canonical_dot(j->x, j->x_is_bf16, j->W, j->K, j->E, m, e, j->kblock, part);
}

void dro_logits(const void *x, int x_is_bf16, const float *W, int64_t M, int64_t K, int64_t E,
                int64_t kblock, float *out, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof(j));
  j.fn = logits_row;
  j.M = M;
  j.x = x;
  j.x_is_bf16 = x_is_bf16;
  j.W = W;
  j.K = K;
  j.E = E;
  j.kblock = kblock;
  j.logits_out = out;
  j.scratch_bytes = (size_t)((K + kblock - 1) / kblock + 1) * sizeof(float);
  run_rows(&j, nthreads);
}

/* ------------------------------------------------------------------ route */

static void route_row(job_t *j, int64_t m, void *scratch) {
  int64_t E = j->E;
  int64_t nb = (j->K + j->kblock - 1) / j->kblock;
  float *raw = (float *)scratch;  /* E */
  float *l = raw + E;             /* E */
  float *u = l + E;               /* 2E */
  float *part = u + 2 * E;        /* nb */
  ent_t *ent = (ent_t *)(part + nb + 1);
  for (int64_t e = 0; e < E; ++e) {
    if (j->split_mode)
      raw[e] = split_dot(j->x, j->x_is_bf16, j->W, j->K, E, m, e, split_factor(j->M));
    else
      raw[e] = canonical_dot(j->x, j->x_is_bf16, j->W, j->K, E, m, e, j->kblock, part);
  }
  route_token(raw, E, j->k, j->logits_bf16, j->flags, l, ent, u, j->ids + m * j->k,
              j->weights ? j->weights + m * j->k : NULL,
              j->sel_logits ? j->sel_logits + m * E : NULL, j->margins ? j->margins + m : NULL);
}

static int route_common(const void *x, int x_is_bf16, const float *W, int64_t M, int64_t K,
                        int64_t E, int32_t k, int64_t kblock, int logits_bf16, uint32_t flags,
                        int32_t *ids, float *weights, float *sel_logits, dro_margin *margins,
                        int nthreads, int split_mode) {
  if (M < 0 || K < 1 || E < 1 || k < 1 || k > E || kblock < 1) return 1;
  if (M > 0 && (!x || !W || !ids)) return 1;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.fn = route_row;
  j.M = M;
  j.x = x;
  j.x_is_bf16 = x_is_bf16;
  j.W = W;
  j.K = K;
  j.E = E;
  j.k = k;
  j.kblock = kblock;
  j.logits_bf16 = logits_bf16;
  j.flags = flags;
  j.split_mode = split_mode;
  j.ids = ids;
  j.weights = weights;
  j.sel_logits = sel_logits;
  j.margins = margins;
  int64_t nb = (K + kblock - 1) / kblock;
  j.scratch_bytes = (size_t)(4 * E + nb + 1) * sizeof(float) + (size_t)E * sizeof(ent_t) + 64;
  run_rows(&j, nthreads);
  return 0;
}

/* ------------------------------------------------------------------ select */

static void select_row(job_t *j, int64_t m, void *scratch) {
  int64_t E = j->E;
  float *l = (float *)scratch; /* E */
  float *u = l + E;            /* 2E */
  ent_t *ent = (ent_t *)(u + 2 * E);
  route_token(j->logits_in + m * E, E, j->k, 0, j->flags, l, ent, u, j->ids + m * j->k,
              j->weights ? j->weights + m * j->k : NULL, NULL, j->margins ? j->margins + m : NULL);
}

int dro_select(const float *logits, int64_t M, int64_t E, int32_t k, uint32_t flags, int32_t *ids,
               float *weights, dro_margin *margins, int nthreads) {
  if (M < 0 || E < 1 || k < 1 || k > E) return 1;
  if (M > 0 && (!logits || !ids)) return 1;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.fn = select_row;
  j.M = M;
  j.E = E;
  j.k = k;
  j.flags = flags;
  j.logits_in = logits;
  j.ids = ids;
  j.weights = weights;
  j.margins = margins;
  j.scratch_bytes = (size_t)(3 * E + 1) * sizeof(float) + (size_t)E * sizeof(ent_t) + 64;
  run_rows(&j, nthreads);
  return 0;
}

int dro_route(const void *x, int x_is_bf16, const float *W, int64_t M, int64_t K, int64_t E,
              int32_t k, int64_t kblock, int logits_bf16, uint32_t flags, int32_t *ids,
              float *weights, float *sel_logits, dro_margin *margins, int nthreads) {
  return route_common(x, x_is_bf16, W, M, K, E, k, kblock, logits_bf16, flags, ids, weights,
                      sel_logits, margins, nthreads, 0);
}

int dro_route_split_by_m(const void *x, int x_is_bf16, const float *W, int64_t M, int64_t K,
                         int64_t E, int32_t k, int logits_bf16, uint32_t flags, int32_t *ids,
                         float *weights, float *sel_logits, dro_margin *margins, int nthreads) {
  return route_common(x, x_is_bf16, W, M, K, E, k, 256, logits_bf16, flags, ids, weights,
                      sel_logits, margins, nthreads, 1);
}

/* ------------------------------------------------------------------ gate */

/* "Batch changed the model's mind", sections "m-scan: the staircase" and "The
 * fix": the shared-expert gate is a one-output dot followed by a sigmoid, and
 * it must be m-invariant like the router.  The dot is the canonical order with
 * E = 1.  Reading for the sigmoid: with e = exp(-|z|) from dro_expf,
 * sigmoid(z) = 1/(1+e) for z >= 0 and e/(1+e) for z < 0 (no overflow). */
static void gate_row(job_t *j, int64_t m, void *scratch) {
  float *part = (float *)scratch;
  int64_t K = j->K;
  int64_t nb = (K + j->kblock - 1) / j->kblock;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t k0 = b * j->kblock, k1 = k0 + j->kblock < K ? k0 + j->kblock : K;
    float p = 0.0f;
    for (int64_t kk = k0; kk < k1; ++kk) {
      float xv = x_at(j->x, j->x_is_bf16, K, m, kk);
      float wv = j->w_is_bf16 ? bf16_widen(((const uint16_t *)j->w)[kk]) : ((const float *)j->w)[kk];
      p = fmaf(xv, wv, p);
    }
    part[b] = p;
  }
  float z = pairwise_tree(part, nb);
  if (j->dot) j->dot[m] = z;
  if (j->gate) {
    float e = dro_expf(-fabsf(z));
    j->gate[m] = (z >= 0.0f) ? 1.0f / (1.0f + e) : e / (1.0f + e);
  }
}

void dro_gate_dot(const void *x, int x_is_bf16, const void *w, int w_is_bf16, int64_t M,
                  int64_t K, int64_t kblock, float *dot, float *gate, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof(j));
  j.fn = gate_row;
  j.M = M;
  j.x = x;
  j.x_is_bf16 = x_is_bf16;
  j.w = w;
  j.w_is_bf16 = w_is_bf16;
  j.K = K;
  j.kblock = kblock;
  j.dot = dot;
  j.gate = gate;
  j.scratch_bytes = (size_t)((K + kblock - 1) / kblock + 1) * sizeof(float);
  run_rows(&j, nthreads);
}

/* ------------------------------------------------------------------ gemm */

static void gemm_row(job_t *j, int64_t m, void *scratch) {
  (void)scratch;
  for (int64_t n = 0; n < j->N; ++n) {
    double s = 0.0;
    for (int64_t kk = 0; kk < j->K; ++kk)
      s += (double)bf16_widen(j->xb[m * j->K + kk]) * (double)bf16_widen(j->Wb[kk * j->N + n]);
    j->out[m * j->N + n] = (float)s;
  }
}

void dro_gemm_bf16_ref(const uint16_t *x, const uint16_t *W, float *out, int64_t M, int64_t K,
                       int64_t N, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof(j));
  j.fn = gemm_row;
  j.M = M;
  j.K = K;
  j.N = N;
  j.xb = x;
  j.Wb = W;
  j.out = out;
  run_rows(&j, nthreads);
}

/* Row p of the grouped product: expert e = expert_of[p], source row
 * src_rows[p] (or p), the same plain definition as gemm_row with W[e]. */
static void grouped_row(job_t *j, int64_t p, void *scratch) {
  (void)scratch;
  const int64_t e = j->expert_of[p];
  const int64_t r = j->src_rows ? j->src_rows[p] : p;
  const uint16_t *We = j->Wb + e * j->K * j->N;
  for (int64_t n = 0; n < j->N; ++n) {
    double s = 0.0;
    for (int64_t kk = 0; kk < j->K; ++kk)
      s += (double)bf16_widen(j->xb[r * j->K + kk]) * (double)bf16_widen(We[kk * j->N + n]);
    j->out[p * j->N + n] = (float)s;
  }
}

int dro_grouped_gemm_bf16_ref(const uint16_t *x, int64_t Mx, const int32_t *rows, const uint16_t *W,
                              const int32_t *offsets, int64_t E, int64_t P, int64_t K, int64_t N,
                              float *out, int nthreads) {
  if (E < 1 || P < 0 || K < 1 || N < 1 || offsets[0] != 0 || offsets[E] != P) return 1;
  for (int64_t e = 0; e < E; ++e)
    if (offsets[e + 1] < offsets[e]) return 1;
  for (int64_t p = 0; p < P; ++p)
    if (rows ? (rows[p] < 0 || rows[p] >= Mx) : (p >= Mx)) return 1;
  int32_t *expert_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
  if (!expert_of) return 1;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) expert_of[p] = (int32_t)e;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.fn = grouped_row;
  j.M = P;
  j.K = K;
  j.N = N;
  j.xb = x;
  j.Wb = W;
  j.out = out;
  j.src_rows = rows;
  j.expert_of = expert_of;
  run_rows(&j, nthreads);
  free(expert_of);
  return 0;
}

/* ------------------------------------------------- permutation, combine */

int dro_moe_permute(const int32_t *ids, int64_t M, int32_t k, int32_t E, int32_t *offsets,
                    int32_t *rows, int32_t *pos) {
  if (M < 0 || k < 1 || E < 1) return 1;
  for (int64_t m = 0; m < M; ++m)
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = ids[m * k + j];
      if (e < 0 || e >= E) return 1;
      for (int32_t i = 0; i < j; ++i)
        if (ids[m * k + i] == e) return 1;
    }
  /* one pass per expert, in expert order; inside it, assignments in token order */
  int64_t p = 0;
  for (int32_t e = 0; e < E; ++e) {
    offsets[e] = (int32_t)p;
    for (int64_t m = 0; m < M; ++m)
      for (int32_t j = 0; j < k; ++j)
        if (ids[m * k + j] == e) {
          rows[p] = (int32_t)m;
          pos[m * k + j] = (int32_t)p;
          ++p;
        }
  }
  offsets[E] = (int32_t)p;
  return 0;
}

void dro_moe_gather(const void *x, int64_t elem_bytes, const int32_t *rows, int64_t P, int64_t D,
                    void *xp) {
  const int64_t row_bytes = elem_bytes * D;
  for (int64_t p = 0; p < P; ++p)
    memcpy((char *)xp + p * row_bytes, (const char *)x + (int64_t)rows[p] * row_bytes, (size_t)row_bytes);
}

static float elem_at(const void *a, int is_bf16, int64_t i) {
  return is_bf16 ? bf16_widen(((const uint16_t *)a)[i]) : ((const float *)a)[i];
}

typedef struct {
  const void *y;
  int y_is_bf16;
  const float *weights;
  const int32_t *ids;
  const int32_t *pos;
  const void *shared;
  int shared_is_bf16;
  const float *gate;
  int32_t k;
  int64_t D;
  float *out;
} combine_job;

static void combine_token(const combine_job *c, int64_t m) {
  /* the slots of token m in ascending (expert id, slot index) */
  int32_t order[64];
  int32_t k = c->k;
  for (int32_t j = 0; j < k; ++j) order[j] = j;
  for (int32_t a = 1; a < k; ++a)
    for (int32_t b = a; b > 0; --b) {
      int32_t s = order[b - 1], t = order[b];
      int32_t es = c->ids[m * k + s], et = c->ids[m * k + t];
      if (es > et || (es == et && s > t)) {
        order[b - 1] = t;
        order[b] = s;
      }
    }
  for (int64_t d = 0; d < c->D; ++d) {
    float acc = 0.0f;
    for (int32_t i = 0; i < k; ++i) {
      int32_t s = order[i];
      float yv = elem_at(c->y, c->y_is_bf16, (int64_t)c->pos[m * k + s] * c->D + d);
      acc = fmaf(c->weights[m * k + s], yv, acc);
    }
    if (c->shared) acc = fmaf(c->gate[m], elem_at(c->shared, c->shared_is_bf16, m * c->D + d), acc);
    c->out[m * c->D + d] = acc;
  }
}

typedef struct {
  const combine_job *c;
  int64_t M;
  int nthreads, tid;
} combine_thread;

static void *combine_main(void *p) {
  combine_thread *t = (combine_thread *)p;
  for (int64_t m = t->tid; m < t->M; m += t->nthreads) combine_token(t->c, m);
  return NULL;
}

int dro_moe_combine(const void *y, int y_is_bf16, const float *weights, const int32_t *ids,
                    const int32_t *pos, int64_t P, const void *shared, int shared_is_bf16,
                    const float *gate, int64_t M, int32_t k, int64_t D, float *out, int nthreads) {
  if (M < 0 || k < 1 || k > 64 || D < 0 || (shared && !gate)) return 1;
  for (int64_t i = 0; i < M * k; ++i)
    if (pos[i] < 0 || pos[i] >= P) return 1;
  combine_job c = {y, y_is_bf16, weights, ids, pos, shared, shared_is_bf16, gate, k, D, out};
  int n = nthreads > 0 ? nthreads : dro_default_threads();
  if (n > 64) n = 64;
  pthread_t th[64];
  combine_thread ct[64];
  for (int i = 0; i < n; ++i) {
    ct[i] = (combine_thread){&c, M, n, i};
    pthread_create(&th[i], NULL, combine_main, &ct[i]);
  }
  for (int i = 0; i < n; ++i) pthread_join(th[i], NULL);
  return 0;
}
