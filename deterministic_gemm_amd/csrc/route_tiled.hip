// route_tiled.hip -- the batched routing kernel on fp32 matrix cores.
//
// gfx950's v_mfma_f32_16x16x1_4b_f32 performs, for four independent 16x16
// blocks, one step acc[i][j] <- fma(a[i], b[j], acc[i][j]) with a single
// rounding: the same operation as one step of the canonical fmaf chain (this
// is checked bit for bit against CPU fmaf chains, subnormals and signed zeros
// included, by the parity tests).  The kernel uses the four blocks of that
// instruction for four consecutive K-blocks of the SAME 16x16 (token, expert)
// tile: slot s of group g runs the chain of K-block 4g+s.  After 256 steps the
// four partials of a tile sit in the same lane, and the first two levels of
// the canonical pairwise tree are lane-local adds; groups are then folded by
// the counter tree.  So every output is produced by exactly the operations of
// the canonical order -- the tile shape and the token count only decide which
// lane performs them ("Batch changed the model's mind", section "The fix:
// m-invariant twins": a batched twin bit-identical per row to the per-row
// kernel is "a perf seam, not a numeric one").
//
// Steps of a chain past the end of K, and slots past the last K-block, are
// fed one zero operand of each sign (x = -0.0 and W = +0.0 in the
// register-staged kernel, the reverse in the pipelined one): the product is
// -0.0 and fma(-0, +0, c) == fma(+0, -0, c) == c for every c, so the padding changes
// no bit; an absent slot starts at -0.0, the identity of the tree's additions.
//
// Work decomposition (E=256): a workgroup of 8 wavefronts takes 32 tokens
// and all E experts; wavefront w owns experts 32w..32w+31 as 2x2 tiles of
// 16x16.  K is walked in chunks of KC steps of all four slots: a chunk of x
// (4 slots x 32 tokens x KC) and of W (4 slots x KC rows x E) is prefetched
// into registers while the previous chunk is consumed from LDS.
#include <type_traits>

#include "route_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace drk {


template <int E_, int AT_, int BT_, int KC_>
struct TiledCfg {
  static constexpr int E = E_;
  static constexpr int AT = AT_;             // 16-token sub-tiles per wavefront
  static constexpr int BT = BT_;             // 16-expert sub-tiles per wavefront
  static constexpr int KC = KC_;             // chain steps per chunk
  static constexpr int EW = 16 * BT;         // experts per wavefront
  static constexpr int NW = E / EW;          // wavefronts per workgroup
  static constexpr int NT = NW * 64;         // threads per workgroup
  static constexpr int TT = 16 * AT;         // tokens per workgroup
  static constexpr int XP = KC + 4;          // x row pitch in LDS (floats)
  static constexpr int XS = 4 * TT * XP;     // x chunk floats
  static constexpr int WSLOT = KC * E + 16;  // W slot stride (floats), +16 staggers banks
  static constexpr int WS = 4 * WSLOT;
  static constexpr int LGP = E + 4;          // logit row pitch for the epilogue
  static constexpr int LDS = (XS + WS > TT * LGP) ? XS + WS : TT * LGP;
  static constexpr int XL = 4 * TT * KC / NT;      // x floats per thread per chunk
  static constexpr int WL = 4 * KC * (E / 4) / NT; // W float4s per thread per chunk
  static constexpr int CPG = 256 / KC;             // chunks per group of 4 K-blocks
  static_assert(XL >= 1 && XL * NT == 4 * TT * KC, "x chunk must split evenly");
  static_assert(WL >= 1 && WL * NT == 4 * KC * (E / 4), "W chunk must split evenly");
  static_assert(KC % 4 == 0 && 256 % KC == 0, "chunk length");
};

template <class C, int MAXL>
__global__ __launch_bounds__(C::NT) void route_tiled_kernel(const float *__restrict__ xf,
                                                            const uint16_t *__restrict__ xb,
                                                            const float *__restrict__ W, int64_t M,
                                                            int K, EpilogueArgs ea) {
  constexpr int E = C::E, AT = C::AT, BT = C::BT, KC = C::KC, TT = C::TT, NT = C::NT;
  __shared__ __attribute__((aligned(16))) float smem[C::LDS];
  float *xs = smem;
  float *ws = smem + C::XS;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int s_l = lane >> 4, r_l = lane & 15;
  const int eb = wave * C::EW;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * TT;
  const int nb = (K + 255) / 256;
  const int G = (nb + 3) / 4;
  const int nchunks = G * C::CPG;

  float xr[C::XL];
  float4 wr[C::WL];

  auto load_chunk = [&](int ci) {
    const int g = ci / C::CPG;
    const int kk0 = (ci % C::CPG) * KC;
#pragma unroll
    for (int i = 0; i < C::XL; ++i) {
      const int idx = t + NT * i;
      const int c = idx % KC, tok = (idx / KC) % TT, s = idx / (KC * TT);
      const int blk = 4 * g + s;
      const int kg = blk * 256 + kk0 + c;
      const int64_t m = m0 + tok;
      float v = -0.0f;
      if (blk < nb && kg < K && m < M) {
        const int64_t off = m * K + kg;
        v = xb ? bf16_to_f32(xb[off]) : xf[off];
      }
      xr[i] = v;
    }
#pragma unroll
    for (int i = 0; i < C::WL; ++i) {
      const int idx = t + NT * i;
      const int e4 = idx % (E / 4), c = (idx / (E / 4)) % KC, s = idx / ((E / 4) * KC);
      const int blk = 4 * g + s;
      const int kg = blk * 256 + kk0 + c;
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (blk < nb && kg < K) v = *reinterpret_cast<const float4 *>(W + static_cast<int64_t>(kg) * E + 4 * e4);
      wr[i] = v;
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < C::XL; ++i) {
      const int idx = t + NT * i;
      const int c = idx % KC, tok = (idx / KC) % TT, s = idx / (KC * TT);
      xs[(s * TT + tok) * C::XP + c] = xr[i];
    }
#pragma unroll
    for (int i = 0; i < C::WL; ++i) {
      const int idx = t + NT * i;
      const int e4 = idx % (E / 4), c = (idx / (E / 4)) % KC, s = idx / ((E / 4) * KC);
      *reinterpret_cast<float4 *>(&ws[s * C::WSLOT + c * E + 4 * e4]) = wr[i];
    }
  };

  f32x16 acc[AT][BT];
  float stk[MAXL][AT * BT * 4];

  load_chunk(0);
  for (int ci = 0; ci < nchunks; ++ci) {
    const int g = ci / C::CPG;
    const int cg = ci % C::CPG;
    if (cg == 0) {
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float init = (4 * g + s < nb) ? 0.0f : -0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[a][b][4 * s + q] = init;
          }
    }
    __syncthreads();
    store_chunk();
    __syncthreads();
    if (ci + 1 < nchunks) load_chunk(ci + 1);

#pragma unroll
    for (int c4 = 0; c4 < KC / 4; ++c4) {
      float4 av[AT];
#pragma unroll
      for (int a = 0; a < AT; ++a)
        av[a] = *reinterpret_cast<const float4 *>(&xs[(s_l * TT + a * 16 + r_l) * C::XP + 4 * c4]);
      float bw[BT][4];
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) bw[b][q] = ws[s_l * C::WSLOT + (4 * c4 + q) * E + eb + b * 16 + r_l];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int a = 0; a < AT; ++a)
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            const float aval = (q == 0) ? av[a].x : (q == 1) ? av[a].y : (q == 2) ? av[a].z : av[a].w;
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x1f32(aval, bw[b][q], acc[a][b], 0, 0, 0);
          }
    }

    if (cg == C::CPG - 1) {
      // levels 1 and 2 of the tree inside the group: (p0 + p1) + (p2 + p3)
      float qv[AT * BT * 4];
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            qv[(a * BT + b) * 4 + q] = (acc[a][b][q] + acc[a][b][4 + q]) + (acc[a][b][8 + q] + acc[a][b][12 + q]);
      tree_push<MAXL, AT * BT * 4>(stk, qv, g);
    }
  }

  float out[AT * BT * 4];
  tree_final<MAXL, AT * BT * 4>(stk, G, out);

  __syncthreads();
  float *lg = smem;
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tok = a * 16 + 4 * s_l + q;
        const int e = eb + b * 16 + r_l;
        lg[tok * C::LGP + e] = out[(a * BT + b) * 4 + q];
      }
  __syncthreads();
  for (int i = 4 * wave; i < TT; i += 4 * C::NW) route_tokens_row16<E>(lg + i * C::LGP, C::LGP, m0 + i, M, ea);
}

// ---------------------------------------------------------------------------
// Pipelined variant for fp32 x with K % 4 == 0: x and W chunks go from global
// memory straight into LDS (global_load_lds_dwordx4: each lane moves 16 bytes,
// written at the instruction's LDS base + 16 * lane) through a ring of S
// stages, so S-1 chunks are in flight while one is consumed and no register
// staging is needed.  Every wavefront issues the same number of transfers per
// chunk (padding transfers read a 16-byte vector of -0.0 or +0.0), so waiting
// for "all but the last (S-2) chunks' transfers" is a fixed vmcnt (one value
// for the wavefronts that also move x, one for the others); a barrier
// after that wait publishes the chunk to all wavefronts and also guarantees
// the stage about to be refilled has been consumed.  The arithmetic per
// output is the same as in route_tiled_kernel above.
//
// LDS stage layout (floats): W rows of slot s at s*SW + c*E (SW = KC*E + 16,
// the 16-float skew spreads the four slot groups over the LDS banks), then x
// as 16-byte units (slot, token, h) with h, the 4-wide piece of the chunk,
// XOR-swizzled by token so that 16 lanes reading one piece of 16 tokens hit
// distinct banks.

template <int E_, int AT_, int BT_, int KC_, int S_>
struct DmaCfg {
  static constexpr int E = E_, AT = AT_, BT = BT_, KC = KC_, S = S_;
  static constexpr int EW = 16 * BT, NW = E / EW, NT = NW * 64, TT = 16 * AT;
  static constexpr int HU = KC / 4;                   // 16-byte units per (slot, token) row
  static constexpr int SW = KC * E + 16;              // W slot stride (floats)
  static constexpr int WST = 4 * SW;                  // W floats per stage
  static constexpr int XST = 4 * TT * KC;             // x floats per stage
  static constexpr int STG = WST + XST;               // floats per stage
  static constexpr int LGP = E + 4;
  static constexpr int WI = 4 * KC * E / 256;         // W transfers (64 lanes x 16 B) per chunk
  static constexpr int WIW = WI / NW;                 // ... per wavefront
  static constexpr int XU = TT * KC;                  // x 16-byte units per chunk
  static constexpr int XI = (XU + 63) / 64;           // x transfers per chunk (64 lanes each) ...
  static constexpr int XW = XI < NW ? XI : NW;        // ... issued by the first XW wavefronts
  static constexpr int XIW = XI / XW;                 // ... XIW each
  static constexpr int PER_X = WIW + XIW;             // transfers per chunk, x-issuing wavefronts
  static constexpr int PER_W = WIW;                   // transfers per chunk, the others
  static constexpr int CPG = 256 / KC;
  static_assert(WIW * NW == WI && WIW >= 1, "W transfers split evenly");
  static_assert(XI * 64 == XU && XIW * XW == XI, "x transfers split evenly");
  static_assert((KC * E / 4) % 64 == 0, "a W transfer stays inside one slot");
  static_assert(PER_X * (S - 1) <= 63, "vmcnt range");
  static_assert(KC % 4 == 0 && 256 % KC == 0 && S >= 2, "chunking");
  __host__ __device__ static constexpr int swz(int tok) { return (tok * HU / 16) % HU; }
};

// Issue the transfers of chunk ci into `stage` (chunks past the end load
// padding, keeping every wavefront's transfer count per chunk fixed).  A
// chunk whose rows are all in range -- every chunk but the K tail, in every
// workgroup but the last -- uses the SGPR-base form; the others address each
// lane separately so that out-of-range lanes can read the padding vectors.
template <class C>
__device__ __forceinline__ void dma_issue(const float *__restrict__ xf, const float *__restrict__ W, int64_t M,
                                          int K, int64_t m0, int nb, int nchunks, int wave, int lane, int ci,
                                          float *stage) {
  constexpr int E = C::E, KC = C::KC, TT = C::TT, HU = C::HU;
  const int g = ci / C::CPG;
  const int kk0 = (ci % C::CPG) * KC;
  const bool live = ci < nchunks;
  // every k of the chunk's four slots is inside K (blocks are 256 apart)
  const bool full_k = live && (4 * g + 3 < nb) && ((4 * g + 3) * 256 + kk0 + KC <= K);
  const bool full_m = m0 + TT <= M;
#pragma unroll
  for (int i = 0; i < C::WIW; ++i) {
    const int j = wave * C::WIW + i;           // transfer index within the chunk
    const int s = j / (KC * E / 256);          // slot
    const int uo = (j % (KC * E / 256)) * 64;  // first 16-byte unit within the slot
    const int u = uo + lane;
    const int c = u / (E / 4), e4 = u % (E / 4);
    const int blk = 4 * g + s;
    const int kg = blk * 256 + kk0 + c;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage + s * C::SW + uo * 4));
    if (full_k) {
      dma16_s(W, static_cast<uint32_t>((kg * E + 4 * e4) * 4), lds);
    } else {
      const void *src = &g_pad_neg;
      if (live && blk < nb && kg < K) src = W + static_cast<int64_t>(kg) * E + 4 * e4;
      dma16(src, lds);
    }
  }
  if (wave < C::XW) {
    const float *xrow0 = xf + m0 * K;  // this workgroup's first row
#pragma unroll
    for (int i = 0; i < C::XIW; ++i) {
      const int u = (wave * C::XIW + i) * 64 + lane;  // x unit within the chunk
      const int s = u / (TT * HU);
      const int rem = u % (TT * HU);
      const int tok = rem / HU, hp = rem % HU;
      const int h = hp ^ C::swz(tok);
      const int blk = 4 * g + s;
      const int kg = blk * 256 + kk0 + 4 * h;
      const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage + C::WST + (wave * C::XIW + i) * 64 * 4));
      if (full_k && full_m) {
        dma16_s(xrow0, static_cast<uint32_t>((tok * K + kg) * 4), lds);
      } else {
        const int64_t m = m0 + tok;
        const void *src = &g_pad_pos;
        if (live && blk < nb && kg < K && m < M) src = xf + m * K + kg;
        dma16(src, lds);
      }
    }
  }
}

// One chunk: retire its transfers, publish them (barrier), refill the stage
// freed by the previous chunk, then 4 slots x KC chain steps on the matrix
// cores; at the end of a group of four K-blocks, fold the group's partials.
template <class C, int MAXL>
__device__ __forceinline__ void dma_step(const float *__restrict__ xf, const float *__restrict__ W, int64_t M,
                                         int K, int64_t m0, int nb, int nchunks, int wave, int lane, int ci,
                                         const float *cur, float *refill, f32x16 (&acc)[C::AT][C::BT],
                                         f32x16 (&stk)[C::AT * C::BT * 4 / 16][MAXL]) {
  constexpr int E = C::E, AT = C::AT, BT = C::BT, KC = C::KC, TT = C::TT, S = C::S, HU = C::HU;
  const int s_l = lane >> 4, r_l = lane & 15;
  const int eb = wave * C::EW;
  const int g = ci / C::CPG;
  const int cg = ci % C::CPG;
  if (cg == 0) {
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float init = (4 * g + s < nb) ? 0.0f : -0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[a][b][4 * s + q] = init;
        }
  }
  compiler_fence();
  if (wave < C::XW)
    wait_vmcnt<C::PER_X * (S - 2)>();
  else
    wait_vmcnt<C::PER_W * (S - 2)>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  dma_issue<C>(xf, W, M, K, m0, nb, nchunks, wave, lane, ci + S - 1, refill);

  const float *xs = cur + C::WST;
#pragma unroll
  for (int c4 = 0; c4 < KC / 4; ++c4) {
    float4 av[AT];
#pragma unroll
    for (int a = 0; a < AT; ++a) {
      const int tok = a * 16 + r_l;
      av[a] = *reinterpret_cast<const float4 *>(xs + ((s_l * TT + tok) * HU + (c4 ^ C::swz(tok))) * 4);
    }
    float bw[BT][4];
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) bw[b][q] = cur[s_l * C::SW + (4 * c4 + q) * E + eb + b * 16 + r_l];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          const float aval = (q == 0) ? av[a].x : (q == 1) ? av[a].y : (q == 2) ? av[a].z : av[a].w;
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x1f32(aval, bw[b][q], acc[a][b], 0, 0, 0);
        }
  }

  if (cg == C::CPG - 1) {
    // levels 1 and 2 of the tree inside the group: (p0 + p1) + (p2 + p3)
    constexpr int NV = AT * BT * 4 / 16;
    static_assert(NV * 16 == AT * BT * 4, "group partials fill whole vectors of 16");
    f32x16 qv[NV];
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int o = (a * BT + b) * 4 + q;
          qv[o / 16][o % 16] = (acc[a][b][q] + acc[a][b][4 + q]) + (acc[a][b][8 + q] + acc[a][b][12 + q]);
        }
#pragma unroll
    for (int v = 0; v < NV; ++v) tree_push_vec<MAXL>(stk[v], qv[v], g);
  }
}

// The S stages are separate __shared__ objects and the chunk loop is unrolled
// by S, so every stage address is a compile-time constant.
template <class C, int MAXL>
__global__ __launch_bounds__(C::NT) void route_tiled_dma_kernel(const float *__restrict__ xf,
                                                                const float *__restrict__ W, int64_t M,
                                                                int K, EpilogueArgs ea) {
  constexpr int E = C::E, AT = C::AT, BT = C::BT, TT = C::TT, S = C::S;
  static_assert(S == 2 || S == 4, "two or four stages");
  __shared__ __attribute__((aligned(16))) float stg0[C::STG];
  __shared__ __attribute__((aligned(16))) float stg1[C::STG];
  __shared__ __attribute__((aligned(16))) float stg2[S == 4 ? C::STG : 4];
  __shared__ __attribute__((aligned(16))) float stg3[S == 4 ? C::STG : 4];
  static_assert(TT * C::LGP <= C::STG, "the epilogue's logits fit in stage 0");

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int s_l = lane >> 4, r_l = lane & 15;
  const int eb = wave * C::EW;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * TT;
  const int nb = (K + 255) / 256;
  const int G = (nb + 3) / 4;
  const int nchunks = G * C::CPG;  // a multiple of S

  f32x16 acc[AT][BT];
  f32x16 stk[AT * BT * 4 / 16][MAXL];

  if constexpr (S == 4) {
    dma_issue<C>(xf, W, M, K, m0, nb, nchunks, wave, lane, 0, stg0);
    dma_issue<C>(xf, W, M, K, m0, nb, nchunks, wave, lane, 1, stg1);
    dma_issue<C>(xf, W, M, K, m0, nb, nchunks, wave, lane, 2, stg2);
    for (int ci = 0; ci < nchunks; ci += 4) {
      dma_step<C, MAXL>(xf, W, M, K, m0, nb, nchunks, wave, lane, ci + 0, stg0, stg3, acc, stk);
      dma_step<C, MAXL>(xf, W, M, K, m0, nb, nchunks, wave, lane, ci + 1, stg1, stg0, acc, stk);
      dma_step<C, MAXL>(xf, W, M, K, m0, nb, nchunks, wave, lane, ci + 2, stg2, stg1, acc, stk);
      dma_step<C, MAXL>(xf, W, M, K, m0, nb, nchunks, wave, lane, ci + 3, stg3, stg2, acc, stk);
    }
  } else {
    dma_issue<C>(xf, W, M, K, m0, nb, nchunks, wave, lane, 0, stg0);
    for (int ci = 0; ci < nchunks; ci += 2) {
      dma_step<C, MAXL>(xf, W, M, K, m0, nb, nchunks, wave, lane, ci + 0, stg0, stg1, acc, stk);
      dma_step<C, MAXL>(xf, W, M, K, m0, nb, nchunks, wave, lane, ci + 1, stg1, stg0, acc, stk);
    }
  }

  f32x16 outv[AT * BT * 4 / 16];
#pragma unroll
  for (int v = 0; v < AT * BT * 4 / 16; ++v) outv[v] = tree_final_vec<MAXL>(stk[v], G);

  // drain the trailing padding transfers before stage 0 is reused for the logits
  compiler_fence();
  wait_vmcnt<0>();
  __syncthreads();
  float *lg = stg0;
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tok = a * 16 + 4 * s_l + q;
        const int e = eb + b * 16 + r_l;
        lg[tok * C::LGP + e] = outv[((a * BT + b) * 4 + q) / 16][((a * BT + b) * 4 + q) % 16];
      }
  __syncthreads();
  for (int i = 4 * wave; i < TT; i += 4 * C::NW) route_tokens_row16<E>(lg + i * C::LGP, C::LGP, m0 + i, M, ea);
}

template <class C, int MAXL>
static hipError_t launch_dma_cm(const RouteLaunch &L) {
  const int64_t nblk = (L.M + C::TT - 1) / C::TT;
  EpilogueArgs ea{L.k, L.logit_bf16, L.flags, L.ids, L.weights, L.logits, L.margins};
  hipLaunchKernelGGL((route_tiled_dma_kernel<C, MAXL>), dim3(static_cast<uint32_t>(nblk)), dim3(C::NT), 0,
                     L.stream, L.xf, L.W, L.M, static_cast<int>(L.K), ea);
  return hipGetLastError();
}

template <class C>
static hipError_t launch_dma_c(const RouteLaunch &L) {
  const int64_t nb = (L.K + 255) / 256;
  const int64_t G = (nb + 3) / 4;
  if (G <= 1) return launch_dma_cm<C, 1>(L);
  if (G <= 2) return launch_dma_cm<C, 2>(L);
  if (G <= 4) return launch_dma_cm<C, 3>(L);
  if (G <= 8) return launch_dma_cm<C, 4>(L);
  return launch_dma_cm<C, 5>(L);
}

template <class C, int MAXL>
static hipError_t launch_tiled_cm(const RouteLaunch &L) {
  const int64_t nblk = (L.M + C::TT - 1) / C::TT;
  EpilogueArgs ea{L.k, L.logit_bf16, L.flags, L.ids, L.weights, L.logits, L.margins};
  hipLaunchKernelGGL((route_tiled_kernel<C, MAXL>), dim3(static_cast<uint32_t>(nblk)), dim3(C::NT), 0, L.stream,
                     L.xf, L.xb, L.W, L.M, static_cast<int>(L.K), ea);
  return hipGetLastError();
}

template <class C>
static hipError_t launch_tiled_c(const RouteLaunch &L) {
  const int64_t nb = (L.K + 255) / 256;
  const int64_t G = (nb + 3) / 4;
  // stack depth = bit length of the number of groups
  if (G <= 1) return launch_tiled_cm<C, 1>(L);
  if (G <= 2) return launch_tiled_cm<C, 2>(L);
  if (G <= 4) return launch_tiled_cm<C, 3>(L);
  if (G <= 8) return launch_tiled_cm<C, 4>(L);
  return launch_tiled_cm<C, 5>(L);
}

bool tiled_supports(int64_t E, int64_t K) {
  return (E == 64 || E == 128 || E == 256 || E == 512) && K >= 1 && K <= 16384;
}

hipError_t launch_route_tiled(const RouteLaunch &L) {
  // fp32 x in whole 16-byte pieces: the pipelined kernel; otherwise (bf16 x,
  // K % 4 != 0) the register-staged one.  Both compute identical bits.
  const bool dma = L.xf != nullptr && (L.K % 4) == 0;
  switch (L.E) {
    case 64: return dma ? launch_dma_c<DmaCfg<64, 2, 2, 8, 4>>(L) : launch_tiled_c<TiledCfg<64, 2, 2, 16>>(L);
    case 128: return dma ? launch_dma_c<DmaCfg<128, 2, 2, 8, 4>>(L) : launch_tiled_c<TiledCfg<128, 2, 2, 16>>(L);
    case 256: return dma ? launch_dma_c<DmaCfg<256, 2, 2, 8, 4>>(L) : launch_tiled_c<TiledCfg<256, 2, 2, 16>>(L);
    case 512: return dma ? launch_dma_c<DmaCfg<512, 1, 4, 4, 4>>(L) : launch_tiled_c<TiledCfg<512, 1, 4, 8>>(L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace drk
