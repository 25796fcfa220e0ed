// route_narrow.hip -- the router's logits for small batches, spread over
// many workgroups.
//
// With few tokens the fused kernel gives one workgroup all E experts and all
// of K, so a handful of CUs stream the whole of W and run every chain step in
// sequence.  Here a workgroup owns a 16*AT-token x 16*BT-expert tile, and its
// KG wavefronts split the groups of four K-blocks between them along the
// canonical tree: with G groups padded to P = 2^ceil(log2 G) leaves, part q
// takes groups [q*P/KG, (q+1)*P/KG) (those below G; a part may be empty), so
// each part is a whole subtree of the canonical tree and
//   logit = the pairwise tree over the KG part values,
// exactly ("The Illusion of Determinism in Disaggregated Inference", section
// "The anatomy of the missing numeric contract": any split that respects the
// stated associative grouping is the same computation).  Inside a part the
// chains, K-block slots, lane-local tree levels and group counter tree are
// those of route_tiled.hip; an empty part is -0.0, the identity of the tree's
// additions, and -0 padding beyond a part's own leaves changes no sum.
//
// Each wavefront streams its own x and W pieces global -> LDS through a
// private ring of S stages (no workgroup barrier in the loop: a wavefront
// reads only what it loaded).  The logits go to the caller's buffer; the
// selection kernel of route_split.hip reads them back.
#include "route_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace drk {

// XB: x holds bf16 bits (K % 8 == 0), staged as they are, 8 values per
// 16-byte unit, and widened exactly when read; else fp32, 4 per unit.
// TX = 8 (with AT = 1): a workgroup takes 8 tokens, staged as 8 rows; the
// matrix steps' rows 8 .. 15 read a 16-byte zero unit at the end of the
// wavefront's ring, so their chains only ever add fmaf(+0, w, .) and are
// never stored.  Twice the workgroups for the same batch, each staging a
// quarter fewer bytes.
template <int E_, int AT_, int BT_, int KG_, int KC_, int S_, bool XB_ = false, int TX_ = 0>
struct NarrowCfg {
  static constexpr int E = E_, AT = AT_, BT = BT_, KG = KG_, KC = KC_, S = S_;
  static constexpr bool XB = XB_;
  static constexpr int XV = XB ? 8 : 4;       // x values per 16-byte unit
  static constexpr int TT = TX_ ? TX_ : 16 * AT, ET = 16 * BT;  // tokens, experts per workgroup
  static_assert(TT == 16 * AT || (AT == 1 && TT == 8), "token rows");
  static constexpr int NT = 64 * KG;
  static constexpr int NET = E / ET;
  static constexpr int HU = KC / XV;          // 16-byte x units per (slot, token) row
  static constexpr int SW = KC * ET + 16;     // W slot stride (floats), +16 staggers banks
  static constexpr int WST = 4 * SW;
  static constexpr int XST = 4 * TT * HU * 4;  // x floats (4-byte words) per stage
  static constexpr int STG = WST + XST;       // floats per stage
  static constexpr int WU = KC * ET / 4;      // W units per slot
  static constexpr int WI = 4 * WU / 64;      // W transfers per chunk
  static constexpr int XI = 4 * TT * HU / 64;  // x transfers per chunk
  static constexpr int PER = WI + XI;
  static constexpr int CPG = 256 / KC;
  static constexpr int NQ = AT * BT * 4;       // group partials per lane
  static_assert(WU % 64 == 0 && WI >= 1 && XI >= 1 && XI * 64 == 4 * TT * HU, "whole transfers");
  static_assert(PER * (S - 1) <= 63 && S >= 2, "vmcnt range");
  static_assert(KC % XV == 0 && 256 % KC == 0, "chunking");
  static_assert(KG == 1 || KG == 2 || KG == 4, "parts");
  static constexpr int RING = S * STG + (TT < 16 * AT ? 4 : 0);  // floats per wavefront (+ the zero unit)
  static_assert((KG * RING + (KG - 1) * 64 * NQ) * 4 <= 160 * 1024, "LDS");
  __host__ __device__ static constexpr int swz(int tok) { return (tok * HU / 16) % HU; }
};

// Transfers of the wave's chunk ci (group g of its part, chunk cg within the
// group) into `stage`; past the wave's last chunk, padding transfers keep the
// count fixed.
template <class C>
__device__ __forceinline__ void narrow_issue(const void *__restrict__ xv, const float *__restrict__ W, int64_t M,
                                             int K, int64_t m0, int e0, int nb, int g0, int nch, int lane, int ci,
                                             float *stage) {
  constexpr int E = C::E, ET = C::ET, KC = C::KC, TT = C::TT, HU = C::HU;
  const bool live = ci < nch;
  const int g = g0 + ci / C::CPG;
  const int kk0 = (ci % C::CPG) * KC;
#pragma unroll
  for (int i = 0; i < C::WI; ++i) {
    const int s = (i * 64) / C::WU;             // slot
    const int uo = (i * 64) % C::WU;            // first unit within the slot
    const int u = uo + lane;
    const int c = u / (ET / 4), e4 = u % (ET / 4);
    const int blk = 4 * g + s;
    const int kg = blk * 256 + kk0 + c;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage + s * C::SW + uo * 4));
    const void *src = &g_pad_neg;
    if (live && blk < nb && kg < K) src = W + static_cast<int64_t>(kg) * E + e0 + 4 * e4;
    dma16(src, lds);
  }
#pragma unroll
  for (int i = 0; i < C::XI; ++i) {
    const int u = i * 64 + lane;
    const int s = u / (TT * HU);
    const int rem = u % (TT * HU);
    const int tok = rem / HU, hp = rem % HU;
    const int h = hp ^ C::swz(tok);
    const int blk = 4 * g + s;
    const int kg = blk * 256 + kk0 + C::XV * h;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage + C::WST + i * 64 * 4));
    const int64_t m = m0 + tok;
    const void *src = &g_pad_pos;
    if (live && blk < nb && kg < K && m < M) src = static_cast<const char *>(xv) + (m * K + kg) * (C::XB ? 2 : 4);
    dma16(src, lds);
  }
}

template <class C, int MAXL>
__global__ __launch_bounds__(C::NT) void route_narrow_logits_kernel(const void *__restrict__ xf,
                                                                    const float *__restrict__ W, int64_t M, int K,
                                                                    void *logits, int logit_bf16) {
  constexpr int ET = C::ET, AT = C::AT, BT = C::BT, TT = C::TT, S = C::S, KC = C::KC, HU = C::HU;
  constexpr int NQ = C::NQ;
  __shared__ __attribute__((aligned(16))) float ring[C::KG * C::RING];
  __shared__ __attribute__((aligned(16))) float parts[C::KG > 1 ? (C::KG - 1) * 64 * NQ : 4];

  const int64_t bid = blockIdx.x;
  const int et = static_cast<int>(bid % C::NET);
  const int64_t m0 = (bid / C::NET) * TT;
  const int e0 = et * ET;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s_l = lane >> 4, r_l = lane & 15;
  const int nb = (K + 255) / 256;
  const int G = (nb + 3) / 4;
  int P = 1;
  while (P < G) P <<= 1;
  const int span = P / C::KG;  // groups per part (P >= KG by the launcher's choice)
  const int g0 = min(G, wave * span), g1 = min(G, (wave + 1) * span);
  const int ng = g1 - g0;
  const int nch = ng * C::CPG;
  float *my = ring + wave * C::RING;
  // rows of the matrix tile past the staged tokens read this zero unit
  [[maybe_unused]] const float *zero = my + S * C::STG;
  if constexpr (TT < 16 * AT) {
    if (lane < 4) my[S * C::STG + lane] = 0.0f;
  }

  f32x16 acc[AT][BT];
  float stk[MAXL][NQ];

#pragma unroll
  for (int i = 0; i < S - 1; ++i) narrow_issue<C>(xf, W, M, K, m0, e0, nb, g0, nch, lane, i, my + i * C::STG);

  for (int ci = 0; ci < nch; ++ci) {
    const int gi = ci / C::CPG, cg = ci % C::CPG;
    const int g = g0 + gi;
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
    wait_vmcnt<C::PER * (S - 2)>();
    compiler_fence();
    narrow_issue<C>(xf, W, M, K, m0, e0, nb, g0, nch, lane, ci + S - 1, my + ((ci + S - 1) % S) * C::STG);
    const float *cur = my + (ci % S) * C::STG;
    // operands of step group c4 + 1 read before the matrix steps of c4, and
    // kept there by a scheduling barrier: a wavefront here runs one dependent
    // chain, so a read issued just before its use (where the scheduler puts
    // it when the reads are interleaved one per matrix step, as in
    // route_split.hip's four chains) leaves every step waiting out the LDS
    // latency.  Measured (whole call, K = 2048, E = 256): 17.7-18.3 against
    // 18.9-19.3 us at M = 65-128, 0.2-1.0 us less at M = 256-2048.
    const float *xs = cur + C::WST;
    float4 av[2][AT];
    float bw[2][BT][4];
    [[maybe_unused]] uint4 ux[2][AT];  // bf16 x: one 16-byte unit feeds two step groups
    const auto read_ops = [&](int c4, int r) {
#pragma unroll
      for (int a = 0; a < AT; ++a) {
        const int tok = a * 16 + r_l;
        if constexpr (C::XB) {
          if ((c4 & 1) == 0) {
            const float *src = xs + ((s_l * TT + tok) * HU + ((c4 >> 1) ^ C::swz(tok))) * 4;
            if constexpr (TT < 16 * AT) src = tok < TT ? src : zero;
            ux[(c4 >> 1) & 1][a] = *reinterpret_cast<const uint4 *>(src);
          }
        } else {
          const float *src = xs + ((s_l * TT + tok) * HU + (c4 ^ C::swz(tok))) * 4;
          if constexpr (TT < 16 * AT) src = tok < TT ? src : zero;
          av[r][a] = *reinterpret_cast<const float4 *>(src);
        }
      }
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) bw[r][b][q] = cur[s_l * C::SW + (4 * c4 + q) * ET + b * 16 + r_l];
    };
    read_ops(0, 0);
#pragma unroll
    for (int c4 = 0; c4 < KC / 4; ++c4) {
      const int r = c4 & 1;
      if constexpr (C::XB) {
#pragma unroll
        for (int a = 0; a < AT; ++a) {
          const uint4 u = ux[(c4 >> 1) & 1][a];
          const uint32_t lo = (c4 & 1) ? u.z : u.x, hi = (c4 & 1) ? u.w : u.y;
          av[r][a] = make_float4(u2f(lo << 16), u2f(lo & 0xFFFF0000u), u2f(hi << 16), u2f(hi & 0xFFFF0000u));
        }
      }
      if (c4 + 1 < KC / 4) read_ops(c4 + 1, r ^ 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int a = 0; a < AT; ++a)
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            const float aval = (q == 0) ? av[r][a].x : (q == 1) ? av[r][a].y : (q == 2) ? av[r][a].z : av[r][a].w;
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x1f32(aval, bw[r][b][q], acc[a][b], 0, 0, 0);
          }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (cg == C::CPG - 1) {
      // levels 1 and 2 of the tree inside the group: (p0 + p1) + (p2 + p3)
      float qv[NQ];
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            qv[(a * BT + b) * 4 + q] = (acc[a][b][q] + acc[a][b][4 + q]) + (acc[a][b][8 + q] + acc[a][b][12 + q]);
      tree_push<MAXL, NQ>(stk, qv, gi);
    }
  }
  // no transfer may still be writing this workgroup's LDS past this point
  compiler_fence();
  wait_vmcnt<0>();

  float part[NQ];
  if (ng > 0) {
    tree_final<MAXL, NQ>(stk, ng, part);
  } else {
#pragma unroll
    for (int j = 0; j < NQ; ++j) part[j] = -0.0f;  // an empty part: the tree's identity
  }
  if constexpr (C::KG > 1) {
    // the top levels of the canonical tree: parts combined pairwise in order
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) parts[((wave - 1) * NQ + j) * 64 + lane] = part[j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float p[C::KG];
      p[0] = part[j];
#pragma unroll
      for (int w = 1; w < C::KG; ++w) p[w] = parts[((w - 1) * NQ + j) * 64 + lane];
      if constexpr (C::KG == 2) part[j] = p[0] + p[1];
      else part[j] = (p[0] + p[1]) + (p[2] + p[3]);
    }
  }

  // lane (s_l, r_l) holds token 16a + 4s_l + q at expert e0 + 16b + r_l
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + a * 16 + 4 * s_l + q;
        const float val = part[(a * BT + b) * 4 + q];
        if (m < M && a * 16 + 4 * s_l + q < TT) {
          const int64_t idx = m * C::E + e0 + b * 16 + r_l;
          if (logit_bf16) static_cast<uint16_t *>(logits)[idx] = f32_to_bf16(val);
          else static_cast<float *>(logits)[idx] = val;
        }
      }
}

template <class C, int MAXL>
static hipError_t launch_narrow_cm(const RouteLaunch &L) {
  const int64_t nblk = (L.M + C::TT - 1) / C::TT * C::NET;
  hipLaunchKernelGGL((route_narrow_logits_kernel<C, MAXL>), dim3(static_cast<uint32_t>(nblk)), dim3(C::NT), 0,
                     L.stream, C::XB ? static_cast<const void *>(L.xb) : static_cast<const void *>(L.xf), L.W, L.M,
                     static_cast<int>(L.K), L.logits, L.logit_bf16);
  return hipGetLastError();
}

// groups per part, then the counter-stack depth for that many groups
template <class C>
static hipError_t launch_narrow_c(const RouteLaunch &L) {
  const int64_t nb = (L.K + 255) / 256;
  const int64_t G = (nb + 3) / 4;
  int64_t P = 1;
  while (P < G) P <<= 1;
  const int64_t span = P / C::KG;
  if (span <= 1) return launch_narrow_cm<C, 1>(L);
  if (span <= 2) return launch_narrow_cm<C, 2>(L);
  if (span <= 4) return launch_narrow_cm<C, 3>(L);
  return launch_narrow_cm<C, 4>(L);
}

// With two to four K-groups (1024 < K <= 4096): the smallest of three tiles
// whose workgroups all fit on the CUs at once, two per CU (66-76 KiB of LDS
// each) --
//   16 x 16 tokens x experts: one part per group (two, or four with a
//     two-stage ring);
//   32 x 16: two parts, 16-step chunks, three stages;
//   32 x 32: two parts, 16-step chunks, two stages (also for larger batches).
// A larger tile gives each wavefront two or four independent chains and reads
// fewer operand bytes per product; a smaller one fills the CUs sooner.  Logits
// kernel alone, bits identical across the tiles: K = 2048, E = 256: M = 1024
// 24 us (16 x 16 tiles: 30), 2048 38 us (the split kernels: 44); K = 4096, E =
// 512: M = 240 22 us (four parts with four stages: 31), 512 40 us (59), 1024
// 65 us (115).  More groups keep one part per group and four stages.
// Chunk lengths are chosen so that a token's row piece of a chunk is 64 or
// 128 bytes, which the L2s serve faster than 32-byte pieces: fp32 x takes
// 32 steps on the 8-row and two-part 16 x 16 tiles and 16 on 32 x 32; bf16 x
// (8 values per 16-byte unit) 32 steps on the 8-row and 16 x 16 tiles (three
// stages where two workgroups share a CU), 32 in two stages on 32 x 16, 16 in
// three on 32 x 32.  Whole call, K = 2048, E = 256, bf16 x: M = 300-500
// 17.3-18.1 against 23.3-23.9 us with 16-step chunks, 600 23.3-24.3 against
// 35.2-36.9, 1024 26.3-27.0 against 37.2-37.7, 2048 36.5-37.2 against
// 40.4-40.8.  fp32 x, 32 against 16 steps: M = 65-128 16.9 against 18.0 us,
// 200-400 17.8-18.2 against 18.8-19.3; 32 x 32 tiles, 16 steps in two stages
// against 8 in four: M = 1500 36.0 against 38.5 us, 2048 38.5 against 41.8, K
// = 4096 and E = 512 at M = 600-1000 63.5-64.6 against 68.2-69.4, K = 3072 at
// M = 1500 61.3 against 66.6.
template <int E, bool XB>
static hipError_t launch_narrow_e(const RouteLaunch &L) {
  const int64_t nb = (L.K + 255) / 256;
  const int64_t G = (nb + 3) / 4;
  const auto wgs = [&](int64_t tt, int64_t et) { return (L.M + tt - 1) / tt * (E / et); };
  // 8 x 16 tiles while their workgroups all fit on the CUs at once
  if (G <= 4 && wgs(8, 16) <= device_cus()) {
    if (G == 1) return launch_narrow_c<NarrowCfg<E, 1, 1, 1, 32, 4, XB, 8>>(L);
    if (G == 2) return launch_narrow_c<NarrowCfg<E, 1, 1, 2, 32, 4, XB, 8>>(L);
    return launch_narrow_c<NarrowCfg<E, 1, 1, 4, 32, 3, XB, 8>>(L);
  }
  if (G == 1) return launch_narrow_c<NarrowCfg<E, 1, 1, 1, XB ? 32 : 16, 4, XB>>(L);
  if (G > 4) return launch_narrow_c<NarrowCfg<E, 1, 1, 4, 16, 4, XB>>(L);
  const int64_t slots = 2 * static_cast<int64_t>(device_cus());
  if (wgs(16, 16) <= slots) {
    // three groups take four parts too (the fourth empty): with two, one
    // part runs two groups in sequence (K = 3072, E = 256, M = 100: 30 us)
    if (G >= 3) return launch_narrow_c<NarrowCfg<E, 1, 1, 4, 16, 2, XB>>(L);
    return launch_narrow_c<NarrowCfg<E, 1, 1, 2, 32, XB ? 3 : 2, XB>>(L);
  }
  if (wgs(32, 16) <= slots) return launch_narrow_c<NarrowCfg<E, 2, 1, 2, XB ? 32 : 16, XB ? 2 : 3, XB>>(L);
  return launch_narrow_c<NarrowCfg<E, 2, 2, 2, 16, XB ? 3 : 2, XB>>(L);
}

// The largest batch the narrow family takes before the split kernels: at
// 1024 < K <= 4096 with E in {256, 512}, as long as its 32 x 32 tiles fit on
// the CUs at once (M = 2048 at E = 256, 1024 at E = 512 on 256 CUs; measured
// crossovers at K = 2048 and 4096); 2048 for one K-group at E = 256;
// otherwise 1280, measured at K = 2048, E = 256 with 16 x 16 tiles.
int64_t narrow_max_m(int64_t E, int64_t K) {
  const int64_t nb = (K + 255) / 256;
  const int64_t G = (nb + 3) / 4;
  if (G >= 2 && G <= 4 && (E == 256 || E == 512)) return 2 * static_cast<int64_t>(device_cus()) * 32 / (E / 32);
  // one K-group at E = 256: the two-kernel family cannot split K into parts
  // there and runs a few dozen workgroups (K = 768 and 1024: 45-48 us for
  // M = 1300-2000 against 32-33 with the 16 x 16 tiles; level from ~2300)
  if (G == 1 && E == 256) return 2048;
  return 1280;
}

bool narrow_supports(int64_t E, int64_t K, bool x_f32, bool has_logits) {
  return (E == 64 || E == 128 || E == 256 || E == 512) && K >= 1 && K <= 16384 && (K % (x_f32 ? 4 : 8)) == 0 &&
         has_logits;
}

hipError_t launch_route_narrow_logits(const RouteLaunch &L) {
  switch (L.E) {
    case 64: return L.xf ? launch_narrow_e<64, false>(L) : launch_narrow_e<64, true>(L);
    case 128: return L.xf ? launch_narrow_e<128, false>(L) : launch_narrow_e<128, true>(L);
    case 256: return L.xf ? launch_narrow_e<256, false>(L) : launch_narrow_e<256, true>(L);
    case 512: return L.xf ? launch_narrow_e<512, false>(L) : launch_narrow_e<512, true>(L);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_route_narrow(const RouteLaunch &L) {
  const hipError_t e = launch_route_narrow_logits(L);
  if (e != hipSuccess) return e;
  return launch_route_select(L);
}

}  // namespace drk
