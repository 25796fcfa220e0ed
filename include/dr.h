/*
 * dr.h -- batch-invariant MoE routing on MI355X (gfx950): the C ABI.
 *
 * The problem, as the pages state it ("Batch changed the model's mind",
 * sections "m-scan: the staircase" and "The fix: m-invariant twins"): a MoE
 * router is an fp32 GEMM logits = x[M,K] . W[K,E] feeding top_k(k of E); a
 * GEMM library that picks its split-K factor, tile or reduction order from M
 * makes a token's logits -- and, at a near-tie, its expert set -- depend on
 * how many other tokens share the call.  This library fixes one reduction
 * order per output that no launch parameter can change:
 *
 *   logit[m,e] = T( c_0, ..., c_{nb-1} ),   nb = ceil(K / 256)
 *   c_b        = fmaf chain from +0 over k = 256b, 256b+1, ... (ascending),
 *                c <- fmaf(x[m,k], W[k,e], c)
 *   T          = pairwise tree: adjacent pairs combined level by level, an
 *                odd last element carried up a level unchanged.
 *
 * ("The Illusion of Determinism in Disaggregated Inference", section "The
 * anatomy of the missing numeric contract": accumulator precision and the
 * associative grouping of the K reduction are what a numeric contract must
 * state; dr_contract() reports them.)  Every kernel variant and tile size is a
 * different schedule of exactly these operations, so results are bit-identical
 * for every M, every position of a row in the batch and every variant.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller (the library keeps none
 *    after returning), row-major and contiguous, 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous on that stream and never synchronise the device.
 *  - The library allocates no device memory.  No value is accumulated by an
 *    atomic anywhere: the routing, GEMM and combine kernels use no atomics,
 *    and dr_moe_permute counts integers (expert histograms, presence bits)
 *    with LDS atomic add / or, whose results do not depend on the order in
 *    which the lanes arrive.
 *  - Arguments are validated before any launch; on a non-OK status no kernel
 *    was launched and outputs are untouched.  DR_ERR_DEVICE means a launch
 *    failed; dr_last_error() then holds the HIP error text.
 *  - M == 0 returns DR_OK without launching anything.
 */
#ifndef DR_H
#define DR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Under C++ the enumerations take a fixed 32-bit underlying type, so any int
 * a caller passes is a value of the type and the range checks below are well
 * defined; C sees plain enums of the same size. */
#ifdef __cplusplus
#define DR_ENUM(name) enum name : int32_t
#else
#define DR_ENUM(name) enum name
#endif

typedef DR_ENUM(dr_status) {
  DR_OK = 0,
  DR_ERR_INVALID = 1,      /* NULL required pointer, bad size, k > E, misaligned pointer */
  DR_ERR_UNSUPPORTED = 2,  /* a shape the GPU path does not implement (see each call) */
  DR_ERR_DEVICE = 3        /* a HIP call or launch failed */
} dr_status;

typedef DR_ENUM(dr_dtype) { DR_F32 = 0, DR_BF16 = 1 } dr_dtype;

/* Kernel families for dr_route.  All produce identical bits; AUTO picks one
 * from M and E only.  Forcing one is a test seam, never a numeric switch. */
typedef DR_ENUM(dr_variant) {
  DR_VARIANT_AUTO = 0,
  DR_VARIANT_ROWWISE = 1, /* few tokens per workgroup, vector FMA (small M) */
  DR_VARIANT_TILED = 2,   /* token tiles on fp32 matrix cores, one K=1 MFMA step per fmaf */
  DR_VARIANT_SPLIT = 3,   /* (token, expert) tiles on matrix cores writing the logits, then a
                             selection kernel reading them back; needs E in {256, 512, 1024}, the
                             logits output, and fp32 x with K % 4 == 0 or bf16 x (staged as
                             it is, widened when read) with K % 8 == 0 and K <= 4096 */
  DR_VARIANT_NARROW = 4,  /* small batches: 16-token x 16-expert tiles whose wavefronts split
                             the K groups along the canonical tree, writing the logits, then
                             the selection kernel; needs E <= 512, the logits output, and
                             K % 4 == 0 (fp32 x) or K % 8 == 0 (bf16 x, staged as it is) */
  DR_VARIANT_TINY = 5,    /* a few tokens: each lane runs (expert, K-block) chains on the vector
                             ALUs with the workgroup's W slice in LDS, the blocks combine across
                             lanes, then the selection kernel; needs K % 4 == 0 (fp32 x)
                             or K % 8 == 0 (bf16 x, widened when read), K <= 4096
                             and the logits output */
  DR_VARIANT_FUSED = 6    /* one launch: 32-token x all-E tiles on matrix cores, the split
                             family's pipeline, then the selection inside the same workgroup;
                             the logits output is optional; needs E = 256 and fp32 x with
                             K % 4 == 0 or bf16 x (staged as it is) with K % 8 == 0 and
                             K <= 4096 */
} dr_variant;

/* Divide the k selected weights by their sum (left to right in rank order). */
#define DR_ROUTE_RENORMALIZE 0x1u

/* Per-token margin, 16 bytes (vllm.cpp PR #2556, section "Why a value tap
 * could never have said this": the smallest selected and the largest rejected
 * logit with their raw bf16 bit patterns, and the margin counted in bf16 ULPs
 * under the sign-magnitude total order -- 0 means the same bf16 value). */
typedef struct dr_margin {
  float sel_min;          /* logit of rank k-1 (the value the selection saw)    */
  float rej_max;          /* logit of rank k; -inf when k == E                  */
  uint16_t sel_min_bf16;  /* bf16 RNE bits of sel_min                           */
  uint16_t rej_max_bf16;  /* bf16 RNE bits of rej_max                           */
  int32_t ulps;           /* ord(sel) - ord(rej), ord(b) = b<0x8000 ? b : -(b&0x7FFF);
                             INT32_MAX when k == E                              */
} dr_margin;

/* The numeric contract of this build. */
typedef struct dr_contract_info {
  int32_t version;    /* 1 */
  int32_t kblock;     /* 256: K-block length of each sequential fmaf chain   */
  int32_t tree;       /* 1: level-by-level adjacent pairs, odd element carried */
  int32_t acc_bits;   /* 32: fp32 accumulation everywhere                     */
  int32_t fma;        /* 1: every product-accumulate is one fused multiply-add */
  int32_t exp_id;     /* 1: Cody-Waite, degree-7 Taylor, exact 2^n scale, t<-87 -> 0 */
  int32_t tie_break;  /* 1: equal values rank by ascending expert index       */
  int32_t max_k;      /* largest supported k                                  */
} dr_contract_info;

/*
 * dr_route -- the fused router: logits, top-k, softmax weights, margins.
 *
 *   x        [M,K] activations; DR_F32, or DR_BF16 bits widened exactly to fp32.
 *   W        [K,E] router weight, fp32.
 *   k        experts per token, 1 <= k <= min(E, 32).
 *   logit_dtype  DR_F32: select on the fp32 logits.  DR_BF16: round each
 *            logit to bf16 (RNE) first and select on those values, as an
 *            engine with a bf16 gate does (vllm.cpp PR #2556, section "Why it
 *            is not a defect").
 *   ids      [M,k] int32, required: expert ids in rank order -- larger logit
 *            first, equal logits by ascending expert index (vllm.cpp PR
 *            #2556, summary: the lowest-index tie-break).  NaN ranks last.
 *   weights  [M,k] fp32 or NULL: softmax over all E logits (max-subtracted,
 *            exp as in dr_contract_info.exp_id, denominator summed by the
 *            pairwise tree in expert order, one IEEE division), gathered at
 *            ids; renormalised over the k when flags has DR_ROUTE_RENORMALIZE.
 *   logits   [M,E] of logit_dtype, or NULL: the values the selection saw.
 *            The two-launch families (narrow, split) keep the logits between
 *            their launches in this buffer, so without it the fused families
 *            run: ~75-90 us below M = 48 against ~20 us, and slower for large
 *            M.  A caller that does not need the logits but wants the faster
 *            families passes a buffer anyway (the Python binding does).
 *   margins  [M] or NULL.
 *
 * bf16 x with K % 8 == 0 takes the families fp32 x does (the two-kernel
 * family up to K = 4096), staged as it is and widened when read.  Elsewhere
 * it takes the register-staged families (tiled, row-wise: ~120 us at K =
 * 2048, E = 256 for any M up to 8192 on MI355X); there, widening it first
 * with dr_widen_bf16 and passing DR_F32 gives the same bits through the
 * faster families, and the Python binding does this by itself.
 *
 * Supported: E in {64, 128, 256, 512, 1024}; 1 <= K <= 16384; k <= 32;
 * 0 <= M <= 2^22 tokens per call (larger M is DR_ERR_INVALID).
 * Other shapes return DR_ERR_UNSUPPORTED (no silent change of numeric path).
 */
dr_status dr_route(const void *x, dr_dtype x_dtype, const float *W, int64_t M, int64_t K,
                   int64_t E, int32_t k, dr_dtype logit_dtype, int32_t *ids, float *weights,
                   void *logits, dr_margin *margins, uint32_t flags, void *stream);

/*
 * dr_route_noalloc -- dr_route for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, same bits as dr_route, and the same family
 * choice as dr_route given a logits buffer.  When logits is NULL and that
 * family runs in two launches (tiny, narrow, split), the logits pass between
 * the launches through the library's one static device buffer of 16 MiB
 * (the fp32 logits of 16384 tokens x 256 experts) instead of a caller
 * buffer, so the call neither allocates nor needs a logits buffer; a batch
 * whose logits (M*E*4 bytes, M*E*2 with DR_BF16 logits) exceed it returns
 * DR_ERR_UNSUPPORTED with the sizes in dr_last_error().  With a logits buffer
 * it is dr_route.  Each GPU holds its own copy of the buffer until the process
 * ends (its address is looked up on the first call per device, with that
 * device current); calls on one GPU share it, so calls that overlap on one
 * GPU (two streams, two threads) race.
 */
dr_status dr_route_noalloc(const void *x, dr_dtype x_dtype, const float *W, int64_t M, int64_t K,
                           int64_t E, int32_t k, dr_dtype logit_dtype, int32_t *ids, float *weights,
                           void *logits, dr_margin *margins, uint32_t flags, void *stream);

/* dr_route with the kernel family forced.  Same bits as dr_route. */
dr_status dr_route_variant(const void *x, dr_dtype x_dtype, const float *W, int64_t M,
                           int64_t K, int64_t E, int32_t k, dr_dtype logit_dtype, int32_t *ids,
                           float *weights, void *logits, dr_margin *margins, uint32_t flags,
                           dr_variant variant, void *stream);

/* The family AUTO picks: a function of the call's shape (M, K, E), the x
 * dtype, whether the logits output is requested, and the current device's
 * compute-unit count (which sets how many workgroups run at once, so where
 * one family stops filling the chip).  It never depends on the data, and
 * every family it can pick computes the same bits. */
dr_variant dr_route_auto_variant(int64_t M, int64_t K, int64_t E, dr_dtype x_dtype, int with_logits);

/*
 * dr_route_logits -- the first half of dr_route on its own: the canonical
 * logits [M,E] (fp32, or rounded to bf16 RNE when logit_dtype is DR_BF16),
 * bit-identical to dr_route's logits output.  Runs the logits kernel of the
 * split family (large M, E in {256, 512}) or of the narrow family: fp32 x,
 * K % 4 == 0 and E in {64, 128, 256, 512}, else DR_ERR_UNSUPPORTED.  logits
 * is required.
 */
dr_status dr_route_logits(const float *x, const float *W, int64_t M, int64_t K, int64_t E,
                          dr_dtype logit_dtype, void *logits, void *stream);

/*
 * dr_route_select -- the second half: top-k with the lowest-index tie-break,
 * softmax weights and margins from given logits, exactly as dr_route selects
 * on its own logits ("vllm.cpp PR #2556", summary: the selection is a
 * function of the logit values alone).  logits [M,E] fp32, or bf16 bits
 * (DR_BF16, widened exactly); the values are used as given.  E in {64, 128,
 * 256, 512, 1024}, 1 <= k <= min(E, 32); ids required, weights and margins may
 * be NULL; flags as in dr_route.
 */
dr_status dr_route_select(const void *logits, dr_dtype logit_dtype, int64_t M, int64_t E, int32_t k,
                          int32_t *ids, float *weights, dr_margin *margins, uint32_t flags,
                          void *stream);

/*
 * dr_gate_dot -- shared-expert gate ("Batch changed the model's mind",
 * section "m-scan: the staircase": a one-output dot that must be m-invariant
 * like the router).  dot[m] = the canonical order above with E = 1;
 * gate[m] = sigmoid(dot[m]) = 1/(1+e) for dot >= 0, e/(1+e) otherwise, with
 * e = exp(-|dot|) from the contract's exp.
 *   x [M,K] (f32 or bf16), w [K] (f32 or bf16), dot [M] fp32 or NULL,
 *   gate [M] fp32 or NULL.  1 <= K <= 16384, M <= 2^22.
 */
dr_status dr_gate_dot(const void *x, dr_dtype x_dtype, const void *w, dr_dtype w_dtype,
                      float *dot, float *gate, int64_t M, int64_t K, void *stream);

/*
 * dr_gemm_bf16 -- batch-invariant dense GEMM out[M,N] = x[M,K] . W[K,N] on
 * bf16 matrix cores with fp32 accumulation ("The Illusion of Determinism in
 * Disaggregated Inference", section "The arithmetic cost of batch-invariant
 * kernels": a static reduction order regardless of the input shape).  Every
 * output row is reduced by the same sequence of MFMA instructions over K
 * whatever M is, so rows are bit-identical across M; the order inside one MFMA
 * is the hardware's, so the result is within a tolerance of the exact product,
 * not bit-equal to a CPU fmaf chain.
 *   x [M,K] bf16 bits, W [K,N] bf16 bits, out [M,N] fp32, all row-major,
 *   device memory owned by the caller, 16-byte aligned (else DR_ERR_INVALID).
 *   K % 32 == 0 and N % 128 == 0; K, N <= 2^30 and M <= 65535*128, else
 *   DR_ERR_UNSUPPORTED.  M == 0 returns DR_OK without a launch.  Errors are
 *   reported before anything is launched.
 */
dr_status dr_gemm_bf16(const uint16_t *x, const uint16_t *W, float *out, int64_t M, int64_t K,
                       int64_t N, void *stream);

/*
 * dr_route_bf16_gemm -- the router as a plain bf16 linear layer, the arm
 * vllm.cpp PR #2556 describes for upstream (section "Why it is not a
 * defect": the gate is a bf16 linear layer and the widening to fp32 happens
 * inside the top-k), next to the fp32 canonical router above.
 *   logits[m,e] = bf16_rne(sum_k x[m,k] * W[k,e]) on bf16 matrix cores with
 *   fp32 accumulation (dr_gemm_bf16's instruction sequence, so rows are
 *   bit-identical across M), then dr_route_select on those bf16 logits: top-k
 *   with the lowest-index tie-break, softmax weights, margin.
 *   x [M,K] bf16 bits, W [K,E] bf16 bits, logits [M,E] bf16 out (required),
 *   ids [M,k], weights [M,k] or NULL, margins [M] or NULL.
 *   K % 32 == 0, E in {128, 256, 512, 1024}, k <= 32, else
 *   DR_ERR_UNSUPPORTED.  The logits are the exact product rounded to bf16 up
 *   to the fp32 accumulation's own rounding (the matrix core's internal order
 *   is the hardware's); the selection, weights and margins are exact
 *   functions of them.
 */
dr_status dr_route_bf16_gemm(const uint16_t *x, const uint16_t *W, int64_t M, int64_t K, int64_t E,
                             int32_t k, int32_t *ids, float *weights, uint16_t *logits, dr_margin *margins,
                             uint32_t flags, void *stream);

/*
 * ---- After routing: token permutation and the MoE combine ----
 *
 * vllm.cpp PR #2556, section "Why a value tap could never have said this":
 * the engine's MoE combine is order-invariant over a token's k slots, and the
 * assembled per-slot expert outputs are one axis of the MoE block (its table
 * in section "The measurement").  The pages stop there; the readings below
 * fix the grouping order and the combine's arithmetic so that both are
 * functions of a token's own routing alone.
 *
 * All pointers are caller-owned device memory, 16-byte aligned (else
 * DR_ERR_INVALID); nothing is allocated, kept or synchronised; argument
 * errors are reported before any launch.
 */

/*
 * dr_moe_permute -- group a route's M*k assignments (token m, slot j) ->
 * expert ids[m,j] by expert: experts ascending, and within an expert tokens
 * ascending (the stable grouping in token order).
 *   ids [M,k] int32, each row k distinct experts in [0,E) (as dr_route
 *     writes them).
 *   offsets [E+1] int32 out: expert e owns grouped rows [offsets[e],
 *     offsets[e+1]); offsets[E] = M*k.
 *   rows [M*k] int32 out: rows[p] = the token of grouped row p.
 *   pos [M,k] int32 out: pos[m,j] = the grouped row of assignment (m,j).
 * 1 <= k <= 32, 1 <= E <= 1024 and M*k < 2^31, else DR_ERR_UNSUPPORTED.
 * M == 0 still writes offsets (all zero).  An id outside [0,E) gets pos -1
 * and no grouped row; a row repeating an expert gets in-range but
 * unspecified positions.  Batches of several 512-token chunks run three
 * launches (per-chunk expert histograms, kept in rows until the last launch
 * overwrites it; placement; rows from pos), smaller ones a single launch.
 */
dr_status dr_moe_permute(const int32_t *ids, int64_t M, int32_t k, int32_t E, int32_t *offsets,
                         int32_t *rows, int32_t *pos, void *stream);

/*
 * dr_widen_bf16 -- out[i] = x[i] widened exactly to fp32 for i in [0,n): the
 * bf16 bits become the upper half of the fp32 pattern, the lower half zero
 * (NaN payloads and signed zeros kept).  How bf16 activations reach the
 * LDS-staged router families with unchanged results (dr_route, "x").
 *   x [n] bf16 bits and out [n] fp32, device memory, 16-byte aligned, not
 *   overlapping; both owned by the caller.  n == 0 is a no-op.
 *   DR_ERR_INVALID for n < 0, missing or misaligned pointers.  One launch on
 *   stream; errors of the launch itself are DR_ERR_DEVICE.
 */
dr_status dr_widen_bf16(const uint16_t *x, int64_t n, float *out, void *stream);

/*
 * dr_moe_gather -- xp[p,:] = x[rows[p],:] for p in [0,P): activations in the
 * grouped order, copied bit for bit.
 *   x [M,D] of dtype (f32 or bf16 bits), rows [P] int32, xp [P,D] same dtype.
 *   A rows entry outside [0,M) gives a zero row.  P < 2^31.
 */
dr_status dr_moe_gather(const void *x, dr_dtype dtype, int64_t M, int64_t D, const int32_t *rows,
                        int64_t P, void *xp, void *stream);

/*
 * dr_moe_combine -- out[m,d] from token m's k slots, independent of their
 * order: the slots are taken in ascending expert id (ascending slot index
 * between equal ids) and
 *   acc = +0; for each slot s in that order: acc = fmaf(w[m,s], y[pos[m,s],d], acc)
 * then, with shared given, acc = fmaf(gate[m], shared[m,d], acc); out = acc.
 *   y [P,D] f32 or bf16 (the expert outputs in grouped order), weights [M,k]
 *   f32, ids [M,k] and pos [M,k] int32 (as dr_route and dr_moe_permute write
 *   them), shared [M,D] f32 or bf16 or NULL, gate [M] f32 (required with
 *   shared; dr_gate_dot's gate), out [M,D] f32.
 *   1 <= k <= 32, D >= 1, P >= 1 when M > 0.  A pos entry outside [0,P)
 *   leaves its slot out (outside the contract; nothing is read past y).
 */
dr_status dr_moe_combine(const void *y, dr_dtype y_dtype, int64_t P, const float *weights,
                         const int32_t *ids, const int32_t *pos, const void *shared,
                         dr_dtype shared_dtype, const float *gate, int64_t M, int32_t k, int64_t D,
                         float *out, void *stream);

/*
 * dr_grouped_gemm_bf16 -- batch-invariant grouped expert GEMM on bf16 matrix
 * cores (the expert GEMM is where two engines' MoE outputs part: vllm.cpp PR
 * #2556, section "The measurement").  Expert e owns output rows p in
 * [offsets[e], offsets[e+1]) and
 *   out[p,n] = sum_k x[r,k] * W[e,k,n],  r = rows[p] (or p when rows is NULL)
 * with fp32 accumulation.  Every output row is reduced by dr_gemm_bf16's
 * instruction sequence, so a row's bits depend only on its x row and W[e]:
 * not on the size or position of its group, nor on the batch, and they equal
 * dr_gemm_bf16 of that one row with W[e].
 *   x [Mx,K] bf16 bits (token order with rows, e.g. dr_moe_permute's rows,
 *   which fuses the gather; grouped order without), W [E,K,N] bf16 bits,
 *   offsets [E+1] int32 (as dr_moe_permute writes them: offsets[0] = 0,
 *   non-decreasing, offsets[E] = P), out [P,N] fp32.
 *   K % 32 == 0, N % 128 == 0, 1 <= E <= 1024, P < 2^31 and
 *   T = ceil(P/128) + E <= 65535 and 8 ceil(T/8) (N/128) < 2^32 (the
 *   workgroup count), else DR_ERR_UNSUPPORTED.  A rows entry outside
 *   [0,Mx) reads a zero row.  Inconsistent offsets leave the affected rows
 *   unwritten; nothing is written outside out.
 */
dr_status dr_grouped_gemm_bf16(const uint16_t *x, int64_t Mx, const int32_t *rows, const uint16_t *W,
                               const int32_t *offsets, int64_t E, int64_t P, int64_t K, int64_t N,
                               float *out, void *stream);

void dr_contract(dr_contract_info *out);
const char *dr_status_string(dr_status s);
/* Text of the last failure on the calling thread ("" if none). */
const char *dr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DR_H */
