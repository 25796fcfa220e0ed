// route_common.h -- device-side pieces shared by the routing kernels:
// scalar conversions, the routing exponential, the rank key, the fixed
// reduction tree over K-block partials, and the per-token epilogue (top-k with
// the lowest-index tie-break, softmax weights, margin).
//
// Numeric definitions implemented here (the same readings the pages leave
// open are taken as stated in include/dr.h):
//  * Tree over K-block partials: adjacent pairs level by level, odd element
//    carried up ("The Illusion of Determinism in Disaggregated Inference",
//    section "The anatomy of the missing numeric contract").  Kernels finish
//    blocks in ascending order and fold them with a binary counter: after the
//    b-th partial (0-based) it is merged with as many stored subtrees as b has
//    trailing one bits.  For nb leaves this is the balanced tree over leaves
//    padded with -0.0 to a power of two, which is the level-by-level tree.
//  * Selection on logits with the lowest-index tie-break, margin in bf16 ULPs
//    under the sign-magnitude order (vllm.cpp PR #2556, summary and section
//    "Why a value tap could never have said this").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dr.h"

namespace drk {

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return u2f(static_cast<uint32_t>(b) << 16); }

// Round to nearest even on the 16 dropped bits: adding 0x7FFF plus the kept
// LSB carries into the kept half exactly when the dropped half is above one
// half, or equal to one half with an odd kept half.  NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  const uint32_t u = f2u(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ int32_t bf16_ord(uint16_t b) {
  return (b & 0x8000u) ? -static_cast<int32_t>(b & 0x7FFFu) : static_cast<int32_t>(b);
}

// The routing exponential for t <= 0: n = rint(t*log2 e), r = t - n*ln2 in two
// fused steps (ln2 split high + low), p = degree-7 Taylor polynomial in Horner
// form with fused steps and fp32 coefficients 1/i!, result p * 2^n with 2^n
// built exactly (n >= -126).  t < -87 gives +0; t > 0 or NaN gives NaN.
__device__ __forceinline__ float route_exp(float t) {
  if (!(t <= 0.0f)) return u2f(0x7FC00000u);
  if (t < -87.0f) return 0.0f;
  const float n = __builtin_rintf(t * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e43p-1f, t);
  r = __builtin_fmaf(-n, -0x1.05c61p-29f, r);
  float p = 0x1.a01a02p-13f;                 // 1/7!
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f); // 1/6!
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);  // 1/5!
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);  // 1/4!
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);  // 1/3!
  p = __builtin_fmaf(p, r, 0x1.0p-1f);       // 1/2!
  p = __builtin_fmaf(p, r, 1.0f);            // 1/1!
  p = __builtin_fmaf(p, r, 1.0f);            // 1/0!
  const int ni = static_cast<int>(n);
  return p * u2f(static_cast<uint32_t>(ni + 127) << 23);
}

// Unsigned key whose order is the ranking order of values: NaN lowest (0),
// -0 and +0 equal, otherwise the IEEE order.
__device__ __forceinline__ uint32_t rank_key(float v) {
  uint32_t u = f2u(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- tree

// Fold the partial of block b (0-based, blocks finished in ascending order)
// into the counter stack.  stk[l] holds the sum of a complete subtree of 2^l
// leaves whenever bit l of the number of finished blocks is set.
template <int MAXL, int N>
__device__ __forceinline__ void tree_push(float (&stk)[MAXL][N], float (&p)[N], int b) {
#pragma unroll
  for (int l = 0; l < MAXL; ++l) {
    if (((b >> l) & 1) == 0) {
#pragma unroll
      for (int o = 0; o < N; ++o) stk[l][o] = p[o];
      return;
    }
#pragma unroll
    for (int o = 0; o < N; ++o) p[o] = stk[l][o] + p[o];
  }
}

// After nb blocks: the stored subtrees sit at the set bits of nb; combine them
// from the smallest (rightmost leaves) upward, which is the padded balanced tree.
template <int MAXL, int N>
__device__ __forceinline__ void tree_final(float (&stk)[MAXL][N], int nb, float (&out)[N]) {
  bool have = false;
#pragma unroll
  for (int l = 0; l < MAXL; ++l) {
    if ((nb >> l) & 1) {
#pragma unroll
      for (int o = 0; o < N; ++o) out[o] = have ? stk[l][o] + out[o] : stk[l][o];
      have = true;
    }
  }
}

// ---------------------------------------------------------------- epilogue

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), d, 64);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), d, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

struct EpilogueArgs {
  int k;
  int logit_bf16;
  uint32_t flags;
  int32_t *ids;
  float *weights;
  void *logits;
  dr_margin *margins;
};

// One wavefront routes one token.  `row` holds the token's E canonical fp32
// logits (in LDS).  Lane l owns experts l*V .. l*V+V-1 (V = E/64).
template <int E>
__device__ void route_token(const float *__restrict__ row, int64_t m, const EpilogueArgs &a) {
  constexpr int V = E / 64;
  const int lane = threadIdx.x & 63;
  const int k = a.k;

  float v[V];
  uint32_t key[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    float t = row[lane * V + j];
    if (a.logit_bf16) t = bf16_to_f32(f32_to_bf16(t));
    v[j] = t;
    key[j] = rank_key(t);
  }

  if (a.logits) {
    if (a.logit_bf16) {
      uint16_t *o = static_cast<uint16_t *>(a.logits) + m * E + lane * V;
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = f32_to_bf16(v[j]);
    } else {
      float *o = static_cast<float *>(a.logits) + m * E + lane * V;
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = v[j];
    }
  }

  // Rank rounds: k winners, plus the first rejected value when k < E.
  const int rounds = (k < E) ? k + 1 : k;
  uint32_t avail = (V >= 32) ? 0xFFFFFFFFu : ((1u << V) - 1u);
  float my_val = 0.0f;  // lane r keeps rank r
  int32_t my_id = 0;
  float mx = 0.0f, sel = 0.0f, rej = -__builtin_inff();
  for (int r = 0; r < rounds; ++r) {
    uint32_t bk = 0;
    int bj = -1;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      if (((avail >> j) & 1u) && (bj < 0 || key[j] > bk)) {
        bk = key[j];
        bj = j;
      }
    }
    // larger key first; on equal keys the larger ~index, i.e. the lower index
    uint64_t comp = (bj < 0) ? 0ull
                             : ((static_cast<uint64_t>(bk) << 32) |
                                static_cast<uint32_t>(~static_cast<uint32_t>(lane * V + bj)));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint64_t o = shfl_xor_u64(comp, d);
      comp = (o > comp) ? o : comp;
    }
    const int win = static_cast<int>(~static_cast<uint32_t>(comp));
    const int owner = win / V, wj = win % V;
    float cand = v[0];
#pragma unroll
    for (int j = 1; j < V; ++j) cand = (j == wj) ? v[j] : cand;
    const float wv = __shfl(cand, owner, 64);
    if (lane == owner) avail &= ~(1u << wj);
    if (r < k && lane == r) {
      my_val = wv;
      my_id = win;
    }
    if (r == 0) mx = wv;
    if (r == k - 1) sel = wv;
    if (r == k) rej = wv;
  }

  if (a.weights) {
    float u[V];
#pragma unroll
    for (int j = 0; j < V; ++j) u[j] = route_exp(v[j] - mx);
#pragma unroll
    for (int w = V; w > 1; w >>= 1) {
#pragma unroll
      for (int i = 0; i < w / 2; ++i) u[i] = u[2 * i] + u[2 * i + 1];
    }
    float s = u[0];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) s = s + __shfl_xor(s, d, 64);
    float w = route_exp(my_val - mx) / s;
    if (a.flags & DR_ROUTE_RENORMALIZE) {
      float rs = __shfl(w, 0, 64);
      for (int j = 1; j < k; ++j) rs = rs + __shfl(w, j, 64);
      w = w / rs;
    }
    if (lane < k) a.weights[m * k + lane] = w;
  }
  if (lane < k) a.ids[m * k + lane] = my_id;
  if (a.margins && lane == 0) {
    dr_margin g;
    g.sel_min = sel;
    g.rej_max = rej;
    g.sel_min_bf16 = f32_to_bf16(sel);
    g.rej_max_bf16 = f32_to_bf16(rej);
    g.ulps = (k < E) ? (bf16_ord(g.sel_min_bf16) - bf16_ord(g.rej_max_bf16)) : 0x7FFFFFFF;
    a.margins[m] = g;
  }
}

}  // namespace drk
