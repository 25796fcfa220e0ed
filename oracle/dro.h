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

/* Grouped expert GEMM reference: for each expert e and each grouped row p in
 * [offsets[e], offsets[e+1]), out[p,n] = sum_k x[r,k] * W[e,k,n] with
 * r = rows[p] (or p when rows is NULL), evaluated like dro_gemm_bf16_ref
 * (bf16 inputs, fp64 sum in k order, one rounding to fp32).  x is [Mx,K],
 * W is [E,K,N] (bf16 bits), out is [P,N].  vllm.cpp PR #2556, section "The
 * measurement", finds the grouped expert GEMM, not the router, to be where
 * two arms' MoE outputs part; a batch-invariant one must give every row the
 * same bits whatever the size and position of its group ("The Illusion of
 * Determinism in Disaggregated Inference", section "The arithmetic cost of
 * batch-invariant kernels").  This reference is the plain definition the
 * matrix-core path is compared to within a tolerance.  Returns nonzero on
 * inconsistent offsets or a source row outside [0,Mx). */
int dro_grouped_gemm_bf16_ref(const uint16_t *x, int64_t Mx, const int32_t *rows, const uint16_t *W,
                              const int32_t *offsets, int64_t E, int64_t P, int64_t K, int64_t N,
                              float *out, int nthreads);

/* ---- The step after routing: token permutation and the MoE combine ----
 *
 * Source: vllm.cpp PR #2556, section "Why a value tap could never have said
 * this": the engine's MoE combine is order-invariant over a token's k slots,
 * which is why two arms' selections compare as sets of sorted ids; the
 * assembled per-slot expert outputs are one of the block's four axes (the
 * table in section "The measurement").  The pages do not spell the combine
 * out; the readings taken here are stated next to each function. */

/* Group the M*k routing assignments (token m, slot j) -> expert ids[m,j] by
 * expert.  Reading: experts ascending, and within an expert, tokens
 * ascending (a stable grouping of the assignments in token order).
 * offsets [E+1]: offsets[e] = number of assignments to experts < e, so
 *   expert e owns grouped rows [offsets[e], offsets[e+1]) and offsets[E] = M*k.
 * rows [M*k]: rows[p] = the token of grouped row p.
 * pos [M,k]: pos[m,j] = the grouped row of assignment (m,j).
 * Returns nonzero (and writes nothing) when an id is outside [0,E) or a row
 * repeats an expert. */
int dro_moe_permute(const int32_t *ids, int64_t M, int32_t k, int32_t E, int32_t *offsets,
                    int32_t *rows, int32_t *pos);

/* xp[p,:] = x[rows[p],:] for p in [0,P): the activations in grouped order.
 * Rows are D elements of elem_bytes bytes each, copied bit for bit. */
void dro_moe_gather(const void *x, int64_t elem_bytes, const int32_t *rows, int64_t P, int64_t D,
                    void *xp);

/* out[m,d] for a token's k slots.  Reading: the slots are taken in ascending
 * expert id (ascending slot index between equal ids), and
 *   acc = +0;  for each slot s in that order: acc = fmaf(w[m,s], y[pos[m,s],d], acc)
 * then, when `shared` is given, acc = fmaf(gate[m], shared[m,d], acc) last.
 * The result therefore does not depend on the order of the k slots.  y is
 * [P,D] (f32, or bf16 bits widened exactly), shared is [M,D] (same choice)
 * or NULL, gate [M] (required with shared), out [M,D] f32.
 * Returns nonzero when a pos entry is outside [0,P). */
int dro_moe_combine(const void *y, int y_is_bf16, const float *weights, const int32_t *ids,
                    const int32_t *pos, int64_t P, const void *shared, int shared_is_bf16,
                    const float *gate, int64_t M, int32_t k, int64_t D, float *out, int nthreads);

/* Number of threads nthreads<=0 resolves to. */
int dro_default_threads(void);

#ifdef __cplusplus
}
#endif
#endif
