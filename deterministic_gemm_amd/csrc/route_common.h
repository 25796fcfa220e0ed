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
#include <type_traits>

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
//
// Written without branches: the steps run on t clamped to [-87.5, 0] (equal
// to t wherever their result is used; NaN becomes -87.5) and the out-of-range
// cases are selected at the end, so a wavefront never diverges here.
__device__ __forceinline__ float route_exp(float t) {
  const float tc = __builtin_fminf(__builtin_fmaxf(t, -87.5f), 0.0f);
  const float n = __builtin_rintf(tc * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e43p-1f, tc);
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
  const float e = p * u2f(static_cast<uint32_t>(ni + 127) << 23);
  return (t <= 0.0f) ? ((t < -87.0f) ? 0.0f : e) : u2f(0x7FC00000u);
}

// Unsigned key whose order is the ranking order of values: NaN lowest (0),
// -0 and +0 equal, otherwise the IEEE order.
__device__ __forceinline__ uint32_t rank_key(float v) {
  uint32_t u = f2u(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// rank_key(v) + 1 in fewer steps: adding +0 turns -0 into +0 (and leaves
// every other value, subnormals included, as it is), the sign bit spread by an
// arithmetic shift and or-ed with the top bit is the mask that flips a
// negative value whole and a positive one's top bit, and NaN gets 1.
__device__ __forceinline__ uint32_t select_key(float v) {
  const uint32_t u = f2u(v + 0.0f);
  const uint32_t flip = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u;
  return (v != v) ? 1u : (u ^ flip) + 1u;
}

// Batcher's odd-even merge sort on N = 2^p elements as a list of
// compare-exchange pairs (a < b), built at compile time.
template <int N>
struct OddEvenNet {
  static constexpr int count() {
    int c = 0;
    for (int p = 1; p < N; p <<= 1)
      for (int k = p; k >= 1; k >>= 1)
        for (int j = k % p; j + k < N; j += 2 * k)
          for (int i = 0; i < k && i + j + k < N; ++i)
            if ((i + j) / (2 * p) == (i + j + k) / (2 * p)) ++c;
    return c;
  }
  static constexpr int C = count();
  struct Pairs {
    int a[C > 0 ? C : 1], b[C > 0 ? C : 1];
  };
  static constexpr Pairs make() {
    Pairs t{};
    int c = 0;
    for (int p = 1; p < N; p <<= 1)
      for (int k = p; k >= 1; k >>= 1)
        for (int j = k % p; j + k < N; j += 2 * k)
          for (int i = 0; i < k && i + j + k < N; ++i)
            if ((i + j) / (2 * p) == (i + j + k) / (2 * p)) {
              t.a[c] = i + j;
              t.b[c] = i + j + k;
              ++c;
            }
    return t;
  }
  static constexpr Pairs pairs = make();
};

// Sorts N 64-bit words in descending order, each compare-exchange one 64-bit
// comparison and two selects per word.
template <int N, int I = 0>
__device__ __forceinline__ void sort_desc(uint64_t (&c)[N]) {
  if constexpr (I < OddEvenNet<N>::C) {
    constexpr int a = OddEvenNet<N>::pairs.a[I], b = OddEvenNet<N>::pairs.b[I];
    const uint64_t x = c[a], y = c[b];
    const bool sw = x < y;
    c[a] = sw ? y : x;
    c[b] = sw ? x : y;
    sort_desc<N, I + 1>(c);
  }
}

// ---------------------------------------------------------------- tree

// Fold the partial of block b (0-based, blocks finished in ascending order)
// into the counter stack.  stk[l] holds the sum of a complete subtree of 2^l
// leaves whenever bit l of the number of finished blocks is set.  The level is
// a template parameter so that every stack access has a constant index and
// the stack stays in registers.
template <int L, int MAXL, int N>
__device__ __forceinline__ void tree_push_level(float (&stk)[MAXL][N], float (&p)[N], int b) {
  if constexpr (L < MAXL) {
    if (((b >> L) & 1) == 0) {
#pragma unroll
      for (int o = 0; o < N; ++o) stk[L][o] = p[o];
    } else {
#pragma unroll
      for (int o = 0; o < N; ++o) p[o] = stk[L][o] + p[o];
      tree_push_level<L + 1, MAXL, N>(stk, p, b);
    }
  }
}

template <int MAXL, int N>
__device__ __forceinline__ void tree_push(float (&stk)[MAXL][N], float (&p)[N], int b) {
  tree_push_level<0, MAXL, N>(stk, p, b);
}

// After nb blocks: the stored subtrees sit at the set bits of nb; combine them
// from the smallest (rightmost leaves) upward, which is the padded balanced tree.
template <int L, int MAXL, int N>
__device__ __forceinline__ void tree_final_level(float (&stk)[MAXL][N], int nb, float (&out)[N], bool have) {
  if constexpr (L < MAXL) {
    if ((nb >> L) & 1) {
#pragma unroll
      for (int o = 0; o < N; ++o) out[o] = have ? stk[L][o] + out[o] : stk[L][o];
      have = true;
    }
    tree_final_level<L + 1, MAXL, N>(stk, nb, out, have);
  }
}

template <int MAXL, int N>
__device__ __forceinline__ void tree_final(float (&stk)[MAXL][N], int nb, float (&out)[N]) {
  tree_final_level<0, MAXL, N>(stk, nb, out, false);
}

// The same counter tree over whole vectors of 16 partials (one element per
// output; the additions are elementwise fp32 adds).  Kernels keep their group
// stack as vectors so it stays in registers.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

template <int L, int MAXL>
__device__ __forceinline__ void tree_push_vec_level(f32x16 (&stk)[MAXL], f32x16 &p, int b) {
  if constexpr (L < MAXL) {
    if (((b >> L) & 1) == 0) {
      stk[L] = p;
    } else {
      p = stk[L] + p;
      tree_push_vec_level<L + 1, MAXL>(stk, p, b);
    }
  }
}

template <int MAXL>
__device__ __forceinline__ void tree_push_vec(f32x16 (&stk)[MAXL], f32x16 p, int b) {
  tree_push_vec_level<0, MAXL>(stk, p, b);
}

template <int L, int MAXL>
__device__ __forceinline__ void tree_final_vec_level(f32x16 (&stk)[MAXL], int nb, f32x16 &out, bool have) {
  if constexpr (L < MAXL) {
    if ((nb >> L) & 1) {
      out = have ? stk[L] + out : stk[L];
      have = true;
    }
    tree_final_vec_level<L + 1, MAXL>(stk, nb, out, have);
  }
}

template <int MAXL>
__device__ __forceinline__ f32x16 tree_final_vec(f32x16 (&stk)[MAXL], int nb) {
  f32x16 out = {};
  tree_final_vec_level<0, MAXL>(stk, nb, out, false);
  return out;
}

// ---------------------------------------------------------------- epilogue

struct EpilogueArgs {
  int k;
  int logit_bf16;
  uint32_t flags;
  int32_t *ids;
  float *weights;
  void *logits;
  dr_margin *margins;
};

// DPP controls (gfx9 encoding): quad_perm, row rotate right.
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm:[1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm:[2,3,0,1]
constexpr int DPP_ROW_ROR1 = 0x121;
constexpr int DPP_ROW_ROR2 = 0x122;
constexpr int DPP_ROW_ROR4 = 0x124;
constexpr int DPP_ROW_ROR8 = 0x128;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Maximum of a u32 over the wavefront, returned uniform: rotations inside each
// row of 16 lanes, then the four row results combined.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<DPP_ROW_ROR8>(x));
  x = max(x, dpp_u32<DPP_ROW_ROR4>(x));
  x = max(x, dpp_u32<DPP_ROW_ROR2>(x));
  x = max(x, dpp_u32<DPP_ROW_ROR1>(x));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return max(max(a, b), max(c, d));
}

// Pairwise tree sum of one value per lane in lane order (lane 2i with 2i+1,
// then pairs of pairs, ...), returned uniform.  Levels 1-2 pair lanes inside
// quads (every lane of a quad then holds the quad's sum).  Levels 3-4 use
// row rotations, where lane i reads lane i-4 (then i-8) of its row: lanes
// 4-7 combine quads 0 and 1, lanes 12-15 quads 2 and 3, and lanes 12-15 then
// combine those two halves, so lane 16r+15 holds row r's tree sum.  Levels 5-6
// combine the four rows.  Other lanes hold sums of other groupings, never read.
__device__ __forceinline__ float wave_tree_sum(float s) {
  s = s + dpp_f32<DPP_QUAD_XOR1>(s);
  s = s + dpp_f32<DPP_QUAD_XOR2>(s);
  s = dpp_f32<DPP_ROW_ROR4>(s) + s;
  s = dpp_f32<DPP_ROW_ROR8>(s) + s;
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 63));
  return (r0 + r1) + (r2 + r3);
}

// Inverse of rank_key(v) + 1 for selection keys (0 = taken, 1 = NaN); +0 and
// -0 share a key and come back as +0, which no caller distinguishes.
__device__ __forceinline__ float key_value(uint32_t kp1) {
  const uint32_t kk = kp1 - 1u;
  if (kk == 0u) return u2f(0x7FC00000u);
  return u2f((kk & 0x80000000u) ? (kk & 0x7FFFFFFFu) : ~kk);
}

// One wavefront routes one token.  `row` holds the token's E canonical fp32
// logits (in LDS, 16-byte aligned).  Lane l owns experts l*V .. l*V+V-1.
// Each rank round takes the wavefront maximum of the selection keys, then the
// lowest expert index holding it (ballots per slot, first set lane), and
// retires that entry: larger value first, equal values by ascending index.
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
    key[j] = rank_key(t) + 1u;
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

  const int rounds = (k < E) ? k + 1 : k;
  uint32_t my_key = 0, mx_key = 0;
  int32_t my_id = 0;
  int sel_at = 0, rej_at = -1;  // winning expert index of rank k-1 and rank k
  for (int r = 0; r < rounds; ++r) {
    uint32_t lm = key[0];
#pragma unroll
    for (int j = 1; j < V; ++j) lm = max(lm, key[j]);
    const uint32_t wmax = wave_max_u32(lm);
    int best = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint64_t msk = __builtin_amdgcn_ballot_w64(key[j] == wmax);
      if (msk) best = min(best, static_cast<int>(__builtin_ctzll(msk)) * V + j);
    }
    const int wl = best / V, wj = best % V;
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (j == wj && lane == wl) key[j] = 0u;
    if (lane == r) {
      my_key = wmax;
      my_id = best;
    }
    if (r == 0) mx_key = wmax;
    if (r == k - 1) sel_at = best;
    if (r == k) rej_at = best;
  }

  if (a.weights) {
    const float mx = key_value(mx_key);
    float u[V];
#pragma unroll
    for (int j = 0; j < V; ++j) u[j] = route_exp(v[j] - mx);
#pragma unroll
    for (int w = V; w > 1; w >>= 1) {
#pragma unroll
      for (int i = 0; i < w / 2; ++i) u[i] = u[2 * i] + u[2 * i + 1];
    }
    const float s = wave_tree_sum(u[0]);
    float w = route_exp(key_value(my_key) - mx) / s;
    if (a.flags & DR_ROUTE_RENORMALIZE) {
      float rs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), 0));
      for (int j = 1; j < k; ++j)
        rs = rs + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
      w = w / rs;
    }
    if (lane < k) a.weights[m * k + lane] = w;
  }
  if (lane < k) a.ids[m * k + lane] = my_id;
  if (a.margins) {
    // exact values (sign of zero included) of ranks k-1 and k, read back
    float cs = v[0], cr = v[0];
#pragma unroll
    for (int j = 1; j < V; ++j) {
      cs = (j == sel_at % V) ? v[j] : cs;
      cr = (rej_at >= 0 && j == rej_at % V) ? v[j] : cr;
    }
    const float sel = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cs), sel_at / V));
    float rej = -__builtin_inff();
    if (rej_at >= 0) rej = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cr), rej_at / V));
    if (lane == 0) {
      dr_margin g;
      g.sel_min = sel;
      g.rej_max = rej;
      g.sel_min_bf16 = f32_to_bf16(sel);
      g.rej_max_bf16 = f32_to_bf16(rej);
      g.ulps = (k < E) ? (bf16_ord(g.sel_min_bf16) - bf16_ord(g.rej_max_bf16)) : 0x7FFFFFFF;
      a.margins[m] = g;
    }
  }
}

// Maximum of a u32 over each row of 16 lanes, returned in every lane of the row.
__device__ __forceinline__ uint32_t row_max16(uint32_t x) {
  x = max(x, dpp_u32<DPP_ROW_ROR8>(x));
  x = max(x, dpp_u32<DPP_ROW_ROR4>(x));
  x = max(x, dpp_u32<DPP_ROW_ROR2>(x));
  x = max(x, dpp_u32<DPP_ROW_ROR1>(x));
  return x;
}

// Pairwise tree sum over the 16 lanes of each row in lane order, returned in
// every lane of the row: the same four levels as wave_tree_sum's first four
// (lane 16r+15 ends up with row r's sum), then a broadcast from that lane.
__device__ __forceinline__ float row_tree_sum16(float s) {
  s = s + dpp_f32<DPP_QUAD_XOR1>(s);
  s = s + dpp_f32<DPP_QUAD_XOR2>(s);
  s = dpp_f32<DPP_ROW_ROR4>(s) + s;
  s = dpp_f32<DPP_ROW_ROR8>(s) + s;
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane | 15) << 2, __builtin_bit_cast(int, s)));
}

// Maximum / bitwise or of a lane's N values as a balanced tree (short
// dependency chains).
template <int N>
__device__ __forceinline__ uint32_t lane_max(const uint32_t (&a)[N]) {
  uint32_t t[N];
#pragma unroll
  for (int j = 0; j < N; ++j) t[j] = a[j];
#pragma unroll
  for (int w = N; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) t[i] = max(t[i], t[i + w / 2]);
  return t[0];
}

template <int N>
__device__ __forceinline__ uint32_t lane_or(const uint32_t (&a)[N]) {
  uint32_t t[N];
#pragma unroll
  for (int j = 0; j < N; ++j) t[j] = a[j];
#pragma unroll
  for (int w = N; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) t[i] = t[i] | t[i + w / 2];
  return t[0];
}

// Maximum / pairwise tree sum over each half of 32 lanes, returned in every
// lane of the half: the 16-lane step, then v_permlane16_swap of the value with
// itself, which hands each lane of rows (0, 1) both rows' values as (row 0,
// row 1), likewise rows (2, 3) -- the tree's next level, lower lanes left.
__device__ __forceinline__ uint32_t row_max32(uint32_t x) {
  x = row_max16(x);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return max(static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1]));
}

__device__ __forceinline__ float row_tree_sum32(float s) {
  s = row_tree_sum16(s);
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, s), __builtin_bit_cast(uint32_t, s),
                                                  false, false);
  return __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) + __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}

// Selection, weights and margin for 64/LT tokens per wavefront, one per group
// of LT = 16, 32 or 64 lanes: the same results as route_token; with 16 or 32
// lanes several tokens' rank rounds proceed together, and with 64 a round
// takes a balanced lane maximum and one ballot instead of route_token's
// per-slot ballots.  Lane q of a group holds in v the selection values of
// experts q*V .. q*V+V-1 (V = E/LT) of token m (bf16-rounded already in
// bf16-logit mode); the lane-local tree over V terms and the tree over the
// LT lanes together are the canonical tree over the E terms in index order
// for either LT.  rp is the group's LDS scratch of at least 68 floats:
// [0, 33) the winning ids by rank, [33, 66) their keys (then their weights),
// 66 and 67 the exact values at ranks k-1 and k.  Groups with live == false
// compute but store nothing.  Needs k <= 32.  Thirty-two lanes per token
// give twice the wavefronts of sixteen for the same tokens, to hide more of
// each round's dependent steps.
template <int E, int LT>
__device__ void route_select_rows(const float (&v)[E / LT], float *rp, int64_t m, bool live,
                                  const EpilogueArgs &a) {
  static_assert(LT == 16 || LT == 32 || LT == 64, "lanes per token");
  constexpr int V = E / LT;
  const int lane = threadIdx.x & 63;
  const int q = lane & (LT - 1);
  const auto group_max = [](uint32_t x) -> uint32_t {
    if constexpr (LT == 16) return row_max16(x);
    if constexpr (LT == 32) return row_max32(x);
    x = row_max32(x);
    return max(static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 0)), static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 32)));
  };
  const auto group_sum = [](float x) -> float {
    if constexpr (LT == 16) return row_tree_sum16(x);
    if constexpr (LT == 32) return row_tree_sum32(x);
    return wave_tree_sum(x);
  };
  const int k = a.k;

  // The lowest lane of the group holding the maximum x == rm.
  const auto first_lane = [&](uint32_t x, uint32_t rm) -> bool {
    const uint64_t bal = __builtin_amdgcn_ballot_w64(x == rm);
    if constexpr (LT == 64) {
      return lane == static_cast<int>(__builtin_ctzll(bal));
    } else {
      const uint32_t bits = static_cast<uint32_t>(bal >> (lane & (64 - LT))) & static_cast<uint32_t>((1ull << LT) - 1);
      return q == static_cast<int>(__builtin_ctz(bits));
    }
  };
  // the winner's records for rank r: expert q*V + slot, its key, and from
  // rank k-1 on its exact value, assembled from the values' bits under masks
  // the compiler cannot see through (a select chain over v becomes an
  // indexed read of v, which it serves from LDS addressed by the linear
  // thread id -- read from the dispatch packet in every wavefront)
  const auto record = [&](int r, int slot, uint32_t rm) {
    rp[r] = __builtin_bit_cast(float, q * V + slot);
    rp[33 + r] = __builtin_bit_cast(float, rm);
    if (r >= k - 1) {
      uint32_t e = 0;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        uint32_t mj = (j == slot) ? ~0u : 0u;
        asm volatile("" : "+v"(mj));
        e |= f2u(v[j]) & mj;
      }
      rp[66 + (r - (k - 1))] = u2f(e);
    }
  };
  const int rounds = (k < E) ? k + 1 : k;

  // Up to 16 values per lane: each lane sorts its (key, slot) pairs once --
  // larger key first, equal keys by ascending slot, as one 64-bit word of
  // key and V-1-slot -- so a round compares the lanes' heads and the winner
  // pops its head: the winner is the group's lowest lane whose head is the
  // maximum, and its head is its lowest slot holding that key, which is the
  // larger-value-first, lower-index-first order over the group.  The slots
  // follow the keys as a packed list of log2(V)-bit fields.  With more values
  // per lane a round scans the lane's keys instead.
  constexpr bool SORTED = V >= 2 && V <= 16;
  constexpr int SB = V >= 16 ? 4 : V >= 8 ? 3 : V >= 4 ? 2 : 1;
  using PackT = typename std::conditional<(SB * V > 32), uint64_t, uint32_t>::type;
  uint32_t key[V];
  PackT slots = 0;
  if constexpr (SORTED) {
    uint64_t c[V];
#pragma unroll
    for (int j = 0; j < V; ++j) c[j] = (static_cast<uint64_t>(select_key(v[j])) << 32) | static_cast<uint32_t>(V - 1 - j);
    sort_desc<V>(c);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      key[j] = static_cast<uint32_t>(c[j] >> 32);
      slots |= static_cast<PackT>(static_cast<uint32_t>(c[j])) << (SB * j);
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) key[j] = select_key(v[j]);
  }

  uint32_t lm = SORTED ? key[0] : lane_max<V>(key);
  const uint32_t top = group_max(lm);
  const float mx = key_value(top);

  // softmax denominator: the canonical tree over the E terms in index order
  // is the tree over each lane's V consecutive terms, then over the LT lanes
  float s = 0.0f;
  if (a.weights) {
    float u[V];
#pragma unroll
    for (int j = 0; j < V; ++j) u[j] = route_exp(v[j] - mx);
#pragma unroll
    for (int w = V; w > 1; w >>= 1) {
#pragma unroll
      for (int i = 0; i < w / 2; ++i) u[i] = u[2 * i] + u[2 * i + 1];
    }
    s = group_sum(u[0]);
  }

  uint32_t rm = top;
  if constexpr (SORTED) {
    for (int r = 0; r < rounds; ++r) {
      if (r > 0) rm = group_max(key[0]);
      const bool win = first_lane(key[0], rm);
      if (win) record(r, V - 1 - static_cast<int>(slots & static_cast<PackT>(V - 1)), rm);
      // the pop as bit selects under an all-ones / all-zeros mask the
      // compiler cannot see through: as plain selects it rewrites key[j] as
      // the sorted list indexed by the lane's pop count, a chain of compares
      // and selects per element
      uint32_t wm = win ? ~0u : 0u;
      asm volatile("" : "+v"(wm));
#pragma unroll
      for (int j = 0; j + 1 < V; ++j) key[j] = (key[j + 1] & wm) | (key[j] & ~wm);
      key[V - 1] = key[V - 1] & ~wm;
      slots = win ? static_cast<PackT>(slots >> SB) : slots;
    }
  } else {
    for (int r = 0; r < rounds; ++r) {
      if (r > 0) {
        lm = lane_max<V>(key);
        rm = group_max(lm);
      }
      // the group's lowest lane holding the maximum, then its lowest slot:
      // the slots equal to the maximum as a bit mask, its lowest set bit
      const bool win = first_lane(lm, rm);
      uint32_t hit[V];
#pragma unroll
      for (int j = 0; j < V; ++j) hit[j] = (key[j] == rm) ? (1u << j) : 0u;
      const int li = static_cast<int>(__builtin_ctz(lane_or<V>(hit) | (1u << (V - 1))));
#pragma unroll
      for (int j = 0; j < V; ++j) key[j] = (win && j == li) ? 0u : key[j];
      if (win) record(r, li, rm);
    }
  }

  if (!live) return;
  // ranks j = q, q + LT, ... of the group's token
  for (int j = q; j < k; j += LT) a.ids[m * k + j] = __builtin_bit_cast(int32_t, rp[j]);
  if (a.weights) {
    for (int j = q; j < k; j += LT)
      rp[33 + j] = route_exp(key_value(__builtin_bit_cast(uint32_t, rp[33 + j])) - mx) / s;
    if (a.flags & DR_ROUTE_RENORMALIZE) {
      float rs = rp[33];
      for (int j = 1; j < k; ++j) rs = rs + rp[33 + j];
      for (int j = q; j < k; j += LT) a.weights[m * k + j] = rp[33 + j] / rs;
    } else {
      for (int j = q; j < k; j += LT) a.weights[m * k + j] = rp[33 + j];
    }
  }
  if (a.margins && q == 0) {
    const float sel = rp[66];
    const float rej = (k < E) ? rp[67] : -__builtin_inff();
    dr_margin g;
    g.sel_min = sel;
    g.rej_max = rej;
    g.sel_min_bf16 = f32_to_bf16(sel);
    g.rej_max_bf16 = f32_to_bf16(rej);
    g.ulps = (k < E) ? (bf16_ord(g.sel_min_bf16) - bf16_ord(g.rej_max_bf16)) : 0x7FFFFFFF;
    a.margins[m] = g;
  }
}

// The fused kernels' epilogue: row r of the wavefront takes token m0 + r
// (skipped past M), whose E canonical fp32 logits are at lg + r * pitch in
// LDS (16-byte aligned, pitch >= 68): it stores the token's logits in the
// requested dtype, then selects; the token's LDS row becomes its scratch.
template <int E>
__device__ void route_tokens_row16(float *lg, int pitch, int64_t m0, int64_t M, const EpilogueArgs &a) {
  constexpr int V = E / 16;
  static_assert(V % 4 == 0, "whole float4s per lane");
  const int lane = threadIdx.x & 63;
  const int q = lane & 15, row = lane >> 4;
  const int64_t m = m0 + row;
  const bool live = m < M;
  float *rp = lg + row * pitch;

  float v[V];
#pragma unroll
  for (int j4 = 0; j4 < V / 4; ++j4) {
    const float4 t = *reinterpret_cast<const float4 *>(rp + q * V + 4 * j4);
    v[4 * j4 + 0] = t.x;
    v[4 * j4 + 1] = t.y;
    v[4 * j4 + 2] = t.z;
    v[4 * j4 + 3] = t.w;
  }
  if (a.logit_bf16) {
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = bf16_to_f32(f32_to_bf16(v[j]));
  }

  if (a.logits && live) {
    if (a.logit_bf16) {
      uint32_t pk[V / 2];
#pragma unroll
      for (int j = 0; j < V / 2; ++j)
        pk[j] = static_cast<uint32_t>(f32_to_bf16(v[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * j + 1])) << 16);
      uint32_t *o = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(a.logits) + m * E + q * V);
      if constexpr (V % 8 == 0) {
#pragma unroll
        for (int j = 0; j < V / 8; ++j)
          reinterpret_cast<uint4 *>(o)[j] = make_uint4(pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]);
      } else {
#pragma unroll
        for (int j = 0; j < V / 4; ++j) reinterpret_cast<uint2 *>(o)[j] = make_uint2(pk[2 * j], pk[2 * j + 1]);
      }
    } else {
      float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(a.logits) + m * E + q * V);
#pragma unroll
      for (int j4 = 0; j4 < V / 4; ++j4) o[j4] = make_float4(v[4 * j4], v[4 * j4 + 1], v[4 * j4 + 2], v[4 * j4 + 3]);
    }
  }
  route_select_rows<E, 16>(v, rp, m, live, a);
}

}  // namespace drk
