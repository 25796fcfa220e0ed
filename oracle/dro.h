/*
 * dro.h -- the CPU oracle for batch-invariant MoE routing.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This is a plain, slow, obviously
 * correct host statement of what the routing path computes.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no source, header, table or constant generator with the HIP
 * library in deterministic_gemm_amd/; each side states the arithmetic on its
 * own, so an agreement between the two is evidence, not an echo.
 *
 * Sources (the pages this oracle is written from):
 *  - "Batch changed the model's mind" (tiyuvta.ai blog), sections "m-scan:
 *    the staircase" and "The fix: m-invariant twins": the router is a
 *    256-output F32 GEMV feeding top_k(8 of 256); the fix gives every row a
 *    fixed reduction order that does not depend on how many rows share the
 *    launch.
 *  - "The Illusion of Determinism in Disaggregated Inference" (hiraditya.
 *    github.io), sections "The low-level math of tile shapes" and "The
 *    anatomy of the missing numeric contract": FP32 accumulation and a strict
 *    associative grouping of the K reduction are what a contract must fix.
 *  - vllm.cpp PR #2556, summary and section "Why a value tap could never have
 *    said this": ties at the top-k boundary go to the lowest expert index;
 *    per token, the smallest selected and largest rejected logit, their raw
 *    bf16 bit patterns, and the margin in bf16 ULPs under the sign-magnitude
 *    total order; selection is a function of the logits, not of the
 *    probabilities.
 *
 * Where the pages leave a step open the oracle takes one stated reading
 * (listed next to each function below); the HIP library implements the same
 * readings independently.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no FTZ/DAZ: subnormals are kept on both sides).
 */
#ifndef DRO_H
#define DRO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Per-token margin record, 16 bytes. */
typedef struct dro_margin {
  float sel_min;          /* smallest selected logit (rank k-1)            */
  float rej_max;          /* largest rejected logit (rank k), -inf if k==E */
  uint16_t sel_min_bf16;  /* bf16 RNE bit pattern of sel_min               */
  uint16_t rej_max_bf16;  /* bf16 RNE bit pattern of rej_max               */
  int32_t ulps;           /* ord(sel_bf16) - ord(rej_bf16); INT32_MAX if k==E */
} dro_margin;

/* bf16 round-to-nearest-even of an fp32 value; any NaN -> 0x7FC0. */
uint16_t dro_bf16_rne(float v);

/* Sign-magnitude total order of a bf16 pattern: +x -> x, -x -> -(x & 0x7FFF),
 * so +0 and -0 both map to 0. */
int32_t dro_bf16_ord(uint16_t b);

/* ULP distance a - b under that order. */
int32_t dro_ulps(uint16_t a, uint16_t b);

/* The routing exponential for t <= 0 (Cody-Waite reduction, degree-7 Taylor,
 * exact power-of-two scale).  t < -87 -> +0.  t > 0 or NaN -> quiet NaN. */
float dro_expf(float t);

/* Vectorised dro_expf over n values (for the accuracy sweep). */
void dro_expf_array(const float *t, float *out, int64_t n);

/* Canonical logits: for each (m,e), fp32 fmaf chains from +0 over K-blocks of
 * `kblock` ascending k, combined by the level-by-level pairwise tree.
 * x is [M,K] (f32, or bf16 bits widened exactly when x_is_bf16), W is [K,E]
 * f32, out is [M,E] f32.  nthreads <= 0 means every core of the affinity mask. */
void dro_logits(const void *x, int x_is_bf16, const float *W, int64_t M, int64_t K,
                int64_t E, int64_t kblock, float *out, int nthreads);

/* Full route.  logits_bf16 != 0 rounds each logit to bf16 (RNE) before the
 * selection, softmax and margin.  flags bit 0 = renormalise the k weights.
 * Outputs: ids [M,k] int32 in rank order; weights [M,k] f32 (may be NULL);
 * sel_logits [M,E] f32, the values the selection saw (may be NULL);
 * margins [M] (may be NULL).  Returns 0 on success, nonzero on bad arguments. */
int dro_route(const void *x, int x_is_bf16, const float *W, int64_t M, int64_t K, int64_t E,
              int32_t k, int64_t kblock, int logits_bf16, uint32_t flags, int32_t *ids,
              float *weights, float *sel_logits, dro_margin *margins, int nthreads);

/* Selection alone: the top-k, softmax weights and margins dro_route derives
 * from a row's logits, here from given logits [M,E] f32 used as they are
 * (a bf16-logit caller passes the widened bf16 values).  Same outputs and
 * return convention as dro_route. */
int dro_select(const float *logits, int64_t M, int64_t E, int32_t k, uint32_t flags, int32_t *ids,
               float *weights, dro_margin *margins, int nthreads);

/* POSITIVE CONTROL ONLY (never a product path): like dro_route, but each
 * row's logit is a left-to-right sum of s(M) contiguous K-slices, each a
 * sequential fmaf chain from +0, with s = 1 for M <= 64, 2 for 65 <= M <= 74
 * and 4 for M >= 75 -- a stand-in for a library that switches its split with
 * the batch size.  It must reproduce a staircase over M. */
int dro_route_split_by_m(const void *x, int x_is_bf16, const float *W, int64_t M, int64_t K,
                         int64_t E, int32_t k, int logits_bf16, uint32_t flags, int32_t *ids,
                         float *weights, float *sel_logits, dro_margin *margins, int nthreads);

/* Shared-expert gate: dot[m] = canonical logit with E=1 (x and w f32 or bf16,
 * widened exactly); gate[m] = sigmoid(dot[m]) written through dro_expf. */
void dro_gate_dot(const void *x, int x_is_bf16, const void *w, int w_is_bf16, int64_t M,
                  int64_t K, int64_t kblock, float *dot, float *gate, int nthreads);

/* Dense GEMM reference: out[m,n] = sum_k x[m,k]*W[k,n] with bf16 inputs,
 * evaluated in fp64 (each product is exact in fp64; the sum is sequential in
 * k) and rounded once to fp32.  This is the plain definition the MFMA path is
 * compared to within a tolerance; it does not model any reduction order. */
void dro_gemm_bf16_ref(const uint16_t *x, const uint16_t *W, float *out, int64_t M,
                       int64_t K, int64_t N, int nthreads);

/* Number of threads nthreads<=0 resolves to. */
int dro_default_threads(void);

#ifdef __cplusplus
}
#endif
#endif
