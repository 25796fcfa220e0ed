// route_split.hip -- the router as two kernels, for large batches that also
// ask for the logits.
//
//  1. route_split_logits_kernel: the canonical-order logits GEMM on fp32
//     matrix cores over (token tile, expert tile) workgroups -- 64 tokens x
//     128 experts instead of the fused kernel's 32 x E -- written to the
//     caller's logits buffer in the requested dtype.  A squarer tile moves
//     fewer bytes into LDS per multiply-add: per step of K, 64 + 128 operand
//     values feed 8192 products, against 32 + 256 in the fused kernel.
//  2. route_split_epilogue32_kernel (route_split_epilogue_kernel below 256
//     experts): top-k, softmax weights and margin per token, reading those
//     logits back (two tokens per wavefront; four below 256 experts).
//
// Each output is produced by exactly the operations of the canonical order
// (the same chains, K-block slots, lane-local tree levels and group counter
// tree as the fused kernel, see route_tiled.hip), and the epilogue is the
// fused kernel's, so every result is bit-identical to the fused and row-wise
// kernels for every M ("Batch changed the model's mind", section "The fix:
// m-invariant twins": the tile shape is a performance seam, never a numeric
// one).  In bf16-logit mode the logits are stored rounded and the epilogue
// selects on those stored values, which are the values the fused kernel
// selects on.
#include "route_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace drk {

// A wavefront owns 16*AT tokens x 16*BT experts, as (AT/2) x (BT/2) tiles of
// 32 x 32 for the two-slot matrix instruction.
// With KP = 2 the workgroup's wavefronts form two parts that run the two
// halves of the canonical tree over K-groups (groups padded to P =
// 2^ceil(log2 G) leaves, part q taking groups [qP/2, (q+1)P/2)), each part on
// its own half of every stage; the two part values are added at the end,
// which is the tree's top level, so the logits are the same bits.
// XB: x holds bf16 bits (K % 8 == 0), staged as they are, 8 values per
// 16-byte unit, and widened exactly when read; else fp32, 4 per unit.
template <int E_, int ET_, int AT_, int BT_, int WT_, int KC_, int S_, int KP_ = 1, bool LATE_ = false,
          bool XB_ = false>
struct SplitCfg {
  static constexpr int E = E_, ET = ET_, AT = AT_, BT = BT_, WT = WT_, KC = KC_, S = S_, KP = KP_;
  static constexpr bool LATE = LATE_;  // refill the freed stage after the chunk's matrix steps
  static constexpr bool XB = XB_;
  static_assert(AT % 2 == 0 && BT % 2 == 0, "32 x 32 wavefront sub-tiles");
  static constexpr int XV = XB ? 8 : 4;       // x values per 16-byte unit
  static constexpr int EW = 16 * BT;          // experts per wavefront
  static constexpr int NWE = ET / EW;         // wavefronts across the expert tile
  static constexpr int NWP = NWE * WT;        // wavefronts per part
  static constexpr int NW = NWP * KP;         // wavefronts per workgroup
  static constexpr int NT = NW * 64;          // threads per workgroup
  static constexpr int TW = 16 * AT;          // tokens per wavefront
  static constexpr int TT = WT * TW;          // tokens per workgroup
  static constexpr int NET = E / ET;          // expert tiles
  static constexpr int HU = KC / XV;          // 16-byte x units per (slot, token) row
  static constexpr int SW = KC * ET + 16;     // W slot stride (floats), +16 staggers banks
  static constexpr int WST = 4 * SW;          // W floats per stage and part
  static constexpr int XST = 4 * TT * HU * 4;  // x floats (4-byte words) per stage and part
  static constexpr int PST = WST + XST;       // floats per stage and part
  static constexpr int STG = KP * PST;        // floats per stage
  static constexpr int LGP = ET + 4;          // logit tile pitch (floats)
  static constexpr int WI = 4 * KC * ET / 256;  // W transfers (64 lanes x 16 B) per chunk
  static constexpr int WIW = WI / NWP;          // ... per wavefront of the part
  static constexpr int XU = 4 * TT * HU;        // x 16-byte units per chunk
  static constexpr int XI = XU / 64;            // x transfers per chunk ...
  static constexpr int XW = XI < NWP ? XI : NWP;  // ... issued by the part's first XW wavefronts
  static constexpr int XIW = XI / XW;           // ... XIW each
  static constexpr int PER_X = WIW + XIW;       // transfers per chunk, x-issuing wavefronts
  static constexpr int PER_W = WIW;             // transfers per chunk, the others
  static constexpr int CPG = 256 / KC;          // chunks per group of four K-blocks
  // One expert tile covering all E: a workgroup holds whole tokens and runs
  // the selection itself (one launch)
  static constexpr bool FUSED = ET == E;
  static_assert(NWE * EW == ET, "whole wavefront expert tiles");
  static_assert(WIW * NWP == WI && WIW >= 1, "W transfers split evenly");
  static_assert(XI * 64 == XU && XIW * XW == XI && XIW >= 1, "x transfers split evenly");
  static_assert(KP == 1 || KP == 2, "parts");
  static_assert(!FUSED || (KP == 1 && TT % (4 * NW) == 0 && ET + 4 >= 68), "fused: whole tokens per wavefront row");
  static_assert((KC * ET / 4) % 64 == 0, "a W transfer stays inside one slot");
  static_assert(PER_X * (S - 1) <= 63, "vmcnt range");
  static_assert(KC % XV == 0 && 256 % KC == 0 && S >= 2 && S <= 4, "chunking");
  static_assert(TT * LGP + (KP - 1) * NWP * AT * BT * 4 * 64 <= S * STG, "the logit tile fits in the stages");
  static_assert(E % ET == 0, "whole expert tiles");
  static_assert(S * STG * 4 <= 160 * 1024, "LDS");
  __host__ __device__ static constexpr int swz(int tok) { return (tok * HU / 16) % HU; }
};

// Transfers of chunk ci into `stage`; the same scheme as the fused kernel's
// dma_issue (route_tiled.hip), with W columns e0 .. e0+ET-1 only.
template <class C>
__device__ __forceinline__ void split_issue(const void *__restrict__ xv, const float *__restrict__ W, int64_t M,
                                            int K, int64_t m0, int e0, int nb, int nchunks, int span, int wave,
                                            int lane, int ci, float *stage) {
  constexpr int E = C::E, ET = C::ET, KC = C::KC, TT = C::TT, HU = C::HU;
  const int part = wave / C::NWP;
  wave = wave % C::NWP;
  stage += part * C::PST;
  const int g = part * span + ci / C::CPG;
  const int kk0 = (ci % C::CPG) * KC;
  const bool live = ci < nchunks;
  const bool full_k = live && (4 * g + 3 < nb) && ((4 * g + 3) * 256 + kk0 + KC <= K);
  const bool full_m = m0 + TT <= M;
  const float *Wt = W + e0;
#pragma unroll
  for (int i = 0; i < C::WIW; ++i) {
    const int j = wave * C::WIW + i;            // transfer index within the chunk
    const int s = j / (KC * ET / 256);          // slot
    const int uo = (j % (KC * ET / 256)) * 64;  // first 16-byte unit within the slot
    const int u = uo + lane;
    const int c = u / (ET / 4), e4 = u % (ET / 4);
    const int blk = 4 * g + s;
    const int kg = blk * 256 + kk0 + c;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage + s * C::SW + uo * 4));
    if (full_k) {
      dma16_s(Wt, static_cast<uint32_t>((kg * E + 4 * e4) * 4), lds);
    } else {
      const void *src = &g_pad_neg;
      if (live && blk < nb && kg < K) src = Wt + static_cast<int64_t>(kg) * E + 4 * e4;
      dma16(src, lds);
    }
  }
  // x as stored: fp32 or bf16 bits, XS bytes a value
  constexpr int XS = C::XB ? 2 : 4;
  const char *xb = static_cast<const char *>(xv);
  const char *xrow0 = xb + m0 * K * XS;
  if (wave >= C::XW) return;
#pragma unroll
  for (int i = 0; i < C::XIW; ++i) {
    const int u = (wave * C::XIW + i) * 64 + lane;  // x unit within the chunk
    const int s = u / (TT * HU);
    const int rem = u % (TT * HU);
    const int tok = rem / HU, hp = rem % HU;
    const int h = hp ^ C::swz(tok);
    const int blk = 4 * g + s;
    const int kg = blk * 256 + kk0 + C::XV * h;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage + C::WST + (wave * C::XIW + i) * 64 * 4));
    if (full_k && full_m) {
      dma16_s(reinterpret_cast<const float *>(xrow0), static_cast<uint32_t>((tok * K + kg) * XS), lds);
    } else {
      const int64_t m = m0 + tok;
      const void *src = &g_pad_pos;
      if (live && blk < nb && kg < K && m < M) src = xb + (m * K + kg) * XS;
      dma16(src, lds);
    }
  }
}

// A wavefront's chains: v[a][b][p][r] is slot 2p + r / 16 of the group,
// token 32a + 8 ((r % 16) / 4) + 4 (lane >> 5) + r % 4, expert 32b + (lane &
// 31) -- the output order of v_mfma_f32_32x32x1_2b_f32, whose two blocks are
// two K-block slots.
template <class C>
struct SplitAcc {
  f32x32 v[C::AT / 2][C::BT / 2][2];
};

// A wavefront's operand registers for one step group of four k, two sets
// (the group being multiplied and the next): per pair p of slots, lane l
// holds x at slot 2p + (l >> 5), token tb + 32a + (l & 31) (bf16 x: a whole
// 16-byte unit of 8 values, read at even groups) and W at that slot, expert
// eb + 32b + (l & 31), four k each.
template <class C>
struct SplitOps {
  float4 av[2][C::AT / 2][2];
  float bw[2][C::BT / 2][2][4];
  uint4 ux[2][C::AT / 2][2];
};

// Reads step group c4's operands from a stage (the part's half) into set r.
template <class C>
__device__ __forceinline__ void split_read_ops(const float *cur, int c4, int r, int tb, int eb, int lane,
                                               SplitOps<C> &o) {
  constexpr int ET = C::ET, TT = C::TT, HU = C::HU, A2 = C::AT / 2, B2 = C::BT / 2;
  const float *xs = cur + C::WST;
  const int hl = lane >> 5, il = lane & 31;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int sl = 2 * p + hl;
#pragma unroll
    for (int a = 0; a < A2; ++a) {
      const int tok = tb + a * 32 + il;
      if constexpr (C::XB) {
        if ((c4 & 1) == 0)
          o.ux[(c4 >> 1) & 1][a][p] =
              *reinterpret_cast<const uint4 *>(xs + ((sl * TT + tok) * HU + ((c4 >> 1) ^ C::swz(tok))) * 4);
      } else {
        o.av[r][a][p] = *reinterpret_cast<const float4 *>(xs + ((sl * TT + tok) * HU + (c4 ^ C::swz(tok))) * 4);
      }
    }
#pragma unroll
    for (int b = 0; b < B2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) o.bw[r][b][p][q] = cur[sl * C::SW + (4 * c4 + q) * ET + eb + b * 32 + il];
  }
}

// One chunk, 4 slots x KC chain steps on the matrix cores, at the end of a
// group of four K-blocks folding the group's partials.  Without ROT a chunk
// starts by publishing itself (each wavefront waits for its own transfers,
// then the barrier) and reading its first step group, and after its matrix
// steps refills the stage the previous chunk freed.  With ROT the chunk's
// first step group was read by the previous chunk (or before the loop), and
// its last step group publishes the next chunk first: each wavefront waits
// for its own transfers of chunk ci + 1 and for its reads of this chunk's
// stage, then the barrier makes chunk ci + 1 visible to all and frees this
// chunk's stage; the next chunk's first operands are read while this chunk's
// last matrix steps run, and the freed stage is refilled with chunk ci + S
// after them, so no wavefront waits for an LDS read at the start of a chunk.
// Measured in one process against the plain order (whole call): M = 8192, K
// = 2048, E = 256 82.1 against 83.7 us; K = 6144 217.3 against 226.9; the
// one-launch family 84.6 against 90.4; but bf16 x 93.4 against 89.7 and K =
// 4096, E = 512 (16-step chunks with a three-level counter stack, which then
// spills) 170.3 against 154.1, so those keep the plain order.
//
// Matrix steps: v_mfma_f32_32x32x1_2b_f32, two K-block slots per
// instruction (32 x 32 outputs each); every output still gets one fused
// multiply-add per k onto its slot's chain.  On random fp32 operands this
// form sustains more of the matrix peak than the four-slot 16 x 16 one (132
// against 120 TFLOP/s in a register-operand microbenchmark, 8 wavefronts per
// CU): the chip holds a higher clock for the same work.  The logits kernel
// measured 84.2 against 85.3 us per call at M = 8192, K = 2048, E = 256 (bf16
// x 89.8 against 91.1, K = 4096, E = 512 154.9 against 158.3).  Operands of
// step group c4 + 1 are read from LDS while the matrix steps of c4 run, into
// the second register set, one read after each matrix step; left to itself
// the scheduler reads each step's W values just before their use and waits
// for them every few matrix steps.
template <class C, int MAXL, bool ROT>
__device__ __forceinline__ void split_step(const void *__restrict__ xf, const float *__restrict__ W, int64_t M,
                                           int K, int64_t m0, int e0, int nb, int nchunks, int span, int wave,
                                           int lane, int ci, const float *cur, const float *nxt, float *refill,
                                           SplitAcc<C> &acc, SplitOps<C> &ops_carried,
                                           f32x16 (&stk)[C::AT * C::BT * 4 / 16][MAXL]) {
  // without ROT the operand registers live within the chunk only
  SplitOps<C> ops_local;
  SplitOps<C> &ops = ROT ? ops_carried : ops_local;
  constexpr int AT = C::AT, BT = C::BT, KC = C::KC, S = C::S;
  constexpr int A2 = AT / 2, B2 = BT / 2;
  static_assert(C::LATE && (KC / 4) % 2 == 0, "the chunk's last step group reads into set 0");
  // with ROT the next chunk's first bf16 unit could land in registers this
  // chunk's last group still widens from (8-step chunks)
  static_assert(!(ROT && C::XB), "bf16 x takes the plain order");
  const int part = wave / C::NWP, wp = wave % C::NWP;
  const int tb = (wp / C::NWE) * C::TW;
  const int eb = (wp % C::NWE) * C::EW;
  const int gi = ci / C::CPG;           // group within the part
  const int g = part * span + gi;
  const int cg = ci % C::CPG;
  cur += part * C::PST;
  nxt += part * C::PST;
  if (cg == 0) {
#pragma unroll
    for (int a = 0; a < A2; ++a)
#pragma unroll
      for (int b = 0; b < B2; ++b)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int r = 0; r < 32; ++r) acc.v[a][b][p][r] = (4 * g + 2 * p + r / 16 < nb) ? 0.0f : -0.0f;
  }
  if constexpr (!ROT) {
    // publish this chunk, then read its first step group
    compiler_fence();
    if (wp < C::XW)
      wait_vmcnt<C::PER_X * (S - 2)>();
    else
      wait_vmcnt<C::PER_W * (S - 2)>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    split_read_ops<C>(cur, 0, 0, tb, eb, lane, ops);
  }
#pragma unroll
  for (int c4 = 0; c4 < KC / 4; ++c4) {
    const int r = c4 & 1;
    if (c4 + 1 < KC / 4) {
      split_read_ops<C>(cur, c4 + 1, r ^ 1, tb, eb, lane, ops);
    } else if constexpr (ROT) {
      compiler_fence();
      if (wp < C::XW)
        wait_vmcnt<C::PER_X * (S - 2)>();
      else
        wait_vmcnt<C::PER_W * (S - 2)>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      split_read_ops<C>(nxt, 0, r ^ 1, tb, eb, lane, ops);
    }
    if constexpr (C::XB) {
      // this group's 4 values are half c4 % 2 of the unit, widened exactly
#pragma unroll
      for (int a = 0; a < A2; ++a)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint4 u = ops.ux[(c4 >> 1) & 1][a][p];
          const uint32_t lo = (c4 & 1) ? u.z : u.x, hi = (c4 & 1) ? u.w : u.y;
          ops.av[r][a][p] = make_float4(u2f(lo << 16), u2f(lo & 0xFFFF0000u), u2f(hi << 16), u2f(hi & 0xFFFF0000u));
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int a = 0; a < A2; ++a)
#pragma unroll
        for (int b = 0; b < B2; ++b)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float4 av = ops.av[r][a][p];
            const float aval = (q == 0) ? av.x : (q == 1) ? av.y : (q == 2) ? av.z : av.w;
            acc.v[a][b][p] = __builtin_amdgcn_mfma_f32_32x32x1f32(aval, ops.bw[r][b][p][q], acc.v[a][b][p], 0, 0, 0);
          }
    constexpr int NR = 2 * A2 + 4 * B2, NM = 4 * A2 * B2 * 2;
    constexpr int NI = NR < NM ? NR : NM;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix step
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    if constexpr (NM > NI) __builtin_amdgcn_sched_group_barrier(0x008, NM - NI, 0);
    if constexpr (NR > NI) __builtin_amdgcn_sched_group_barrier(0x100, NR - NI, 0);
  }
  // refill: with ROT this chunk's stage with chunk ci + S, else the stage the
  // previous chunk freed with chunk ci + S - 1
  compiler_fence();
  split_issue<C>(xf, W, M, K, m0, e0, nb, nchunks, span, wave, lane, ROT ? ci + S : ci + S - 1, refill);
  compiler_fence();

  if (cg == C::CPG - 1) {
    // levels 1 and 2 of the tree inside the group: (p0 + p1) + (p2 + p3)
    constexpr int NV = AT * BT * 4 / 16;
    f32x16 qv[NV];
    // vector a * (BT/2) + b holds sub-tile (a, b) in the 32 x 32 lane order
#pragma unroll
    for (int a = 0; a < A2; ++a)
#pragma unroll
      for (int b = 0; b < B2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          qv[a * B2 + b][r] =
              (acc.v[a][b][0][r] + acc.v[a][b][0][16 + r]) + (acc.v[a][b][1][r] + acc.v[a][b][1][16 + r]);
#pragma unroll
    for (int v = 0; v < NV; ++v) tree_push_vec<MAXL>(stk[v], qv[v], gi);
  }
}

// Workgroup -> (token tile, expert tile).  Workgroups are placed on the eight
// XCDs in turn, so the NET expert tiles of one token tile are given block
// indices eight apart: they land on the same XCD and share its L2, and x is
// fetched from HBM once.  Blocks past the last token tile exit at once.
template <class C, int MAXL>
__global__ __launch_bounds__(C::NT) void route_split_logits_kernel(const void *__restrict__ xf,
                                                                   const float *__restrict__ W, int64_t M, int K,
                                                                   EpilogueArgs ea) {
  constexpr int ET = C::ET, AT = C::AT, BT = C::BT, TT = C::TT, S = C::S, STG = C::STG;
  __shared__ __attribute__((aligned(16))) float smem[S * STG];

  const int64_t bid = blockIdx.x;
  const int64_t hi = bid / 8;
  const int et = static_cast<int>(hi % C::NET);
  const int64_t tt = (hi / C::NET) * 8 + bid % 8;
  const int64_t m0 = tt * TT;
  if (m0 >= M) return;
  const int e0 = et * ET;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int part = wave / C::NWP, wp = wave % C::NWP;
  const int tb = (wp / C::NWE) * C::TW;
  const int eb = (wp % C::NWE) * C::EW;
  const int nb = (K + 255) / 256;
  const int G = (nb + 3) / 4;
  int P = 1;
  while (P < G) P <<= 1;
  // groups per part: all G with one part; half the padded tree with two (the
  // launcher uses two parts only when G >= 2; groups past G are padding)
  const int span = C::KP == 1 ? G : P / 2;
  const int nchunks = span * C::CPG;

  SplitAcc<C> acc;
  f32x16 stk[AT * BT * 4 / 16][MAXL];

  SplitOps<C> ops;
  constexpr bool ROT = !C::XB && !(C::KC == 16 && MAXL >= 3);
  if constexpr (ROT) {
    // all S stages in flight; chunk 0 published and its first operands read
#pragma unroll
    for (int i = 0; i < S; ++i) split_issue<C>(xf, W, M, K, m0, e0, nb, nchunks, span, wave, lane, i, smem + i * STG);
    compiler_fence();
    if (wp < C::XW)
      wait_vmcnt<C::PER_X * (S - 1)>();
    else
      wait_vmcnt<C::PER_W * (S - 1)>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    split_read_ops<C>(smem + part * C::PST, 0, 0, tb, eb, lane, ops);
  } else {
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      split_issue<C>(xf, W, M, K, m0, e0, nb, nchunks, span, wave, lane, i, smem + i * STG);
  }
  // unrolled by S so that every stage address is a compile-time constant
  for (int ci = 0; ci < nchunks; ci += S) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (ci + j < nchunks)
        split_step<C, MAXL, ROT>(xf, W, M, K, m0, e0, nb, nchunks, span, wave, lane, ci + j, smem + j * STG,
                                 smem + ((j + 1) % S) * STG, smem + (ROT ? j : (j + S - 1) % S) * STG, acc, ops,
                                 stk);
  }

  constexpr int NV = AT * BT * 4 / 16;
  f32x16 outv[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) outv[v] = tree_final_vec<MAXL>(stk[v], span);

  // drain the trailing padding transfers, then stage the tile for row stores
  compiler_fence();
  wait_vmcnt<0>();
  __syncthreads();
  float *lg = smem;
  if constexpr (C::KP == 2) {
    // the tree's top level: part 0's value + part 1's value
    float *comb = smem + TT * C::LGP;
    if (part == 1) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < 16; ++j) comb[((wp * NV + v) * 16 + j) * 64 + lane] = outv[v][j];
    }
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < 16; ++j) outv[v][j] = outv[v][j] + comb[((wp * NV + v) * 16 + j) * 64 + lane];
    }
  }
  // vector a * (BT/2) + b, element r: token tb + 32a + 8 (r / 4) + 4 (lane
  // >> 5) + r % 4 at expert eb + 32b + (lane & 31)
  if (part == 0) {
#pragma unroll
    for (int a = 0; a < AT / 2; ++a)
#pragma unroll
      for (int b = 0; b < BT / 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = tb + a * 32 + 8 * (r / 4) + 4 * (lane >> 5) + r % 4;
          lg[tok * C::LGP + eb + b * 32 + (lane & 31)] = outv[a * (BT / 2) + b][r];
        }
  }
  __syncthreads();
  if constexpr (C::FUSED) {
    // whole tokens: each row of 16 lanes selects one token from its LDS row
    // (and stores its logits when asked)
    for (int i = 4 * wave; i < TT; i += 4 * C::NW) route_tokens_row16<C::E>(lg + i * C::LGP, C::LGP, m0 + i, M, ea);
    return;
  }
  if (!ea.logit_bf16) {
    float *out = static_cast<float *>(ea.logits);
    for (int u = t; u < TT * ET / 4; u += C::NT) {
      const int tok = u / (ET / 4), c4 = u % (ET / 4);
      const int64_t m = m0 + tok;
      if (m < M)
        *reinterpret_cast<float4 *>(out + m * C::E + e0 + 4 * c4) =
            *reinterpret_cast<const float4 *>(lg + tok * C::LGP + 4 * c4);
    }
  } else {
    uint16_t *out = static_cast<uint16_t *>(ea.logits);
    for (int u = t; u < TT * ET / 8; u += C::NT) {
      const int tok = u / (ET / 8), c8 = u % (ET / 8);
      const int64_t m = m0 + tok;
      if (m < M) {
        const float *src = lg + tok * C::LGP + 8 * c8;
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pk[j] = static_cast<uint32_t>(f32_to_bf16(src[2 * j])) |
                  (static_cast<uint32_t>(f32_to_bf16(src[2 * j + 1])) << 16);
        *reinterpret_cast<uint4 *>(out + m * C::E + e0 + 8 * c8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      }
    }
  }
}

// Four tokens per wavefront, 16 per workgroup: each row of 16 lanes reads
// its token's logits (as stored: fp32, or bf16 widened exactly) and runs the
// fused kernels' selection epilogue.
template <int E>
__global__ __launch_bounds__(256) void route_split_epilogue_kernel(int64_t M, EpilogueArgs ea) {
  constexpr int V = E / 16;
  __shared__ __attribute__((aligned(16))) float scr[16][68];
  const int t = threadIdx.x;
  const int lane = t & 63, q = lane & 15;
  const int slot = t >> 4;  // wavefront * 4 + row
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 16 + slot;
  const bool live = m < M;
  float v[V];
  if (live) {
    if (ea.logit_bf16) {
      const uint16_t *src = static_cast<const uint16_t *>(ea.logits) + m * E + q * V;
      uint32_t p[V / 2];
      if constexpr (V % 8 == 0) {
#pragma unroll
        for (int j8 = 0; j8 < V / 8; ++j8) {
          const uint4 w = reinterpret_cast<const uint4 *>(src)[j8];
          p[4 * j8 + 0] = w.x;
          p[4 * j8 + 1] = w.y;
          p[4 * j8 + 2] = w.z;
          p[4 * j8 + 3] = w.w;
        }
      } else {
#pragma unroll
        for (int j4 = 0; j4 < V / 4; ++j4) {
          const uint2 w = reinterpret_cast<const uint2 *>(src)[j4];
          p[2 * j4 + 0] = w.x;
          p[2 * j4 + 1] = w.y;
        }
      }
#pragma unroll
      for (int j = 0; j < V / 2; ++j) {
        v[2 * j] = u2f(p[j] << 16);
        v[2 * j + 1] = u2f(p[j] & 0xFFFF0000u);
      }
    } else {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(ea.logits) + m * E + q * V);
#pragma unroll
      for (int j4 = 0; j4 < V / 4; ++j4) {
        const float4 w = src[j4];
        v[4 * j4 + 0] = w.x;
        v[4 * j4 + 1] = w.y;
        v[4 * j4 + 2] = w.z;
        v[4 * j4 + 3] = w.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = 0.0f;
  }
  route_select_rows<E, 16>(v, scr[slot], m, live, ea);
}

// The same with two tokens per wavefront (32 lanes each, eight tokens per
// workgroup): twice the wavefronts, to hide more of each round's latency.
template <int E>
__global__ __launch_bounds__(256) void route_split_epilogue32_kernel(int64_t M, EpilogueArgs ea) {
  constexpr int V = E / 32;
  static_assert(V % 8 == 0, "whole 16-byte loads per lane");
  __shared__ __attribute__((aligned(16))) float scr[8][68];
  const int t = threadIdx.x;
  const int lane = t & 63, q = lane & 31;
  const int slot = t >> 5;  // wavefront * 2 + half
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 8 + slot;
  const bool live = m < M;
  float v[V];
  if (live) {
    if (ea.logit_bf16) {
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(ea.logits) + m * E + q * V);
#pragma unroll
      for (int j8 = 0; j8 < V / 8; ++j8) {
        const uint4 w = src[j8];
        const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * j8 + 2 * j] = u2f(p[j] << 16);
          v[8 * j8 + 2 * j + 1] = u2f(p[j] & 0xFFFF0000u);
        }
      }
    } else {
      const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(ea.logits) + m * E + q * V);
#pragma unroll
      for (int j4 = 0; j4 < V / 4; ++j4) {
        const float4 w = src[j4];
        v[4 * j4 + 0] = w.x;
        v[4 * j4 + 1] = w.y;
        v[4 * j4 + 2] = w.z;
        v[4 * j4 + 3] = w.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = 0.0f;
  }
  route_select_rows<E, 32>(v, scr[slot], m, live, ea);
}

// Small batches: one wavefront per token, which finishes a token in fewer
// dependent steps than several tokens sharing a wavefront; four tokens per
// workgroup.  The token's logits are widened into an LDS row first; the
// selection then sees the values as given and writes no logits.  From 256
// experts, route_select_rows on all 64 lanes (each lane sorts its values
// once, a round is a wavefront maximum of the lanes' heads and one ballot):
// selection alone at E = 256, k = 8 4.0 against 4.3 us at M = 1 and 4.6
// against 4.7-4.8 at M = 64-1024 for route_token's per-slot ballots, which
// fewer experts keep.
template <int E>
__global__ __launch_bounds__(256) void route_select_wave_kernel(int64_t M, EpilogueArgs ea) {
  __shared__ __attribute__((aligned(16))) float rows[4][E + 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (m >= M) return;
  float *row = rows[wave];
  for (int e = lane; e < E; e += 64)
    row[e] = ea.logit_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(ea.logits)[m * E + e])
                           : static_cast<const float *>(ea.logits)[m * E + e];
  __builtin_amdgcn_wave_barrier();
  EpilogueArgs a = ea;
  a.logits = nullptr;
  a.logit_bf16 = 0;
  if constexpr (E >= 256) {
    constexpr int V = E / 64;
    float v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = row[lane * V + j];
    route_select_rows<E, 64>(v, row, m, true, a);  // the row becomes the token's scratch
  } else {
    route_token<E>(row, m, a);
  }
}

template <class C, int MAXL>
static hipError_t launch_logits_cm(const RouteLaunch &L) {
  const int64_t ntt = (L.M + C::TT - 1) / C::TT;
  const int64_t nblk = (ntt + 7) / 8 * 8 * C::NET;
  EpilogueArgs ea{L.k, L.logit_bf16, L.flags, L.ids, L.weights, L.logits, L.margins};
  hipLaunchKernelGGL((route_split_logits_kernel<C, MAXL>), dim3(static_cast<uint32_t>(nblk)), dim3(C::NT), 0,
                     L.stream, C::XB ? static_cast<const void *>(L.xb) : static_cast<const void *>(L.xf), L.W, L.M,
                     static_cast<int>(L.K), ea);
  return hipGetLastError();
}

// LMAX: the deepest counter stack this configuration is launched with.
template <class C, int LMAX = 5>
static hipError_t launch_logits_c(const RouteLaunch &L) {
  const int64_t nb = (L.K + 255) / 256;
  const int64_t G = (nb + 3) / 4;
  int64_t P = 1;
  while (P < G) P <<= 1;
  const int64_t span = C::KP == 1 ? G : P / 2;
  // stack depth = bit length of the number of groups a part folds
  if (span <= 1) return launch_logits_cm<C, 1>(L);
  if (span <= 2) return launch_logits_cm<C, 2>(L);
  if (span <= 4 || LMAX <= 3) return launch_logits_cm<C, LMAX < 3 ? LMAX : 3>(L);
  if constexpr (LMAX >= 4) {
    if (span <= 8) return launch_logits_cm<C, 4>(L);
  }
  return launch_logits_cm<C, LMAX>(L);
}

// Batches up to this size select with one wavefront per token.
constexpr int64_t kSelectWaveMaxM = 1024;

template <int E>
static hipError_t launch_select_e(const RouteLaunch &L) {
  EpilogueArgs ea{L.k, L.logit_bf16, L.flags, L.ids, L.weights, L.logits, L.margins};
  if constexpr (E <= 512) {
    if (L.M > kSelectWaveMaxM) {
      // two tokens per wavefront from 256 experts (8 per lane): measured 158.6
      // against 162.2 us at M = 4096, K = 4096, E = 512, k = 10 and 50.8
      // against 51.6 at M = 4096, K = 2048, E = 256, level at M = 8192
      if constexpr (E >= 256) {
        hipLaunchKernelGGL((route_split_epilogue32_kernel<E>), dim3(static_cast<uint32_t>((L.M + 7) / 8)), dim3(256), 0,
                           L.stream, L.M, ea);
        return hipGetLastError();
      }
      hipLaunchKernelGGL((route_split_epilogue_kernel<E>), dim3(static_cast<uint32_t>((L.M + 15) / 16)), dim3(256), 0,
                         L.stream, L.M, ea);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((route_select_wave_kernel<E>), dim3(static_cast<uint32_t>((L.M + 3) / 4)), dim3(256), 0,
                     L.stream, L.M, ea);
  return hipGetLastError();
}

bool split_supports(int64_t E, int64_t K, bool x_f32, bool has_logits) {
  // bf16 x: the configurations of K <= 4096 (their x transfers divide
  // evenly over the wavefronts at 8 values per unit)
  return (E == 256 || E == 512 || E == 1024) && K >= 1 && K <= (x_f32 ? 16384 : 4096) && (K % (x_f32 ? 4 : 8)) == 0 &&
         has_logits;
}

bool select_supports(int64_t E) { return E == 64 || E == 128 || E == 256 || E == 512 || E == 1024; }

hipError_t launch_route_logits(const RouteLaunch &L) {
  // 64 x 64 tiles with the K-groups split between two parts while that many
  // workgroups still fit the chip in one round (twice the workgroups of the
  // 64 x 128 tiles); needs at least two K-groups.
  const int64_t two_part_wgs = (L.M + 63) / 64 * (L.E / 64);
  const bool two = L.K > 1024 && two_part_wgs <= device_cus();
  switch (L.E) {
    // chunk length, stage count and refill order as measured fastest; chunks
    // of 16 steps need too many registers for the deeper counter stacks of
    // K > 4096.  The two-part 64 x 64 tiles take 16-step chunks (x row pieces
    // of 64 bytes for fp32, 32 for bf16) in two stages (three for bf16 x):
    // 48.7 against 49.4 us at M = 4096, K = 2048, E = 256 for 8-step chunks in
    // four stages (bf16 x 51.4 against 52.1), E = 512 and 1024 0.5-1.7 us less
    case 256:
      if (!L.xf) {
        if (two) return launch_logits_c<SplitCfg<256, 64, 2, 2, 2, 16, 3, 2, true, true>>(L);
        return launch_logits_c<SplitCfg<256, 128, 2, 2, 2, 16, 3, 1, true, true>, 3>(L);
      }
      if (two) return launch_logits_c<SplitCfg<256, 64, 2, 2, 2, 16, 2, 2, true, false>>(L);
      if (L.K > 4096) return launch_logits_c<SplitCfg<256, 128, 2, 2, 2, 8, 4, 1, true, false>>(L);
      return launch_logits_c<SplitCfg<256, 128, 2, 2, 2, 16, 3, 1, true, false>, 3>(L);
    case 512:
      if (!L.xf) {
        if (two) return launch_logits_c<SplitCfg<512, 64, 2, 2, 2, 16, 3, 2, true, true>>(L);
        return launch_logits_c<SplitCfg<512, 128, 2, 2, 2, 16, 3, 1, true, true>, 3>(L);
      }
      if (two) return launch_logits_c<SplitCfg<512, 64, 2, 2, 2, 16, 2, 2, true, false>>(L);
      if (L.K > 4096) return launch_logits_c<SplitCfg<512, 128, 2, 2, 2, 8, 4, 1, true, false>>(L);
      return launch_logits_c<SplitCfg<512, 128, 2, 2, 2, 16, 3, 1, true, false>, 3>(L);
    case 1024:
      if (!L.xf) {
        if (two) return launch_logits_c<SplitCfg<1024, 64, 2, 2, 2, 16, 3, 2, true, true>>(L);
        return launch_logits_c<SplitCfg<1024, 128, 2, 2, 2, 16, 3, 1, true, true>, 3>(L);
      }
      if (two) return launch_logits_c<SplitCfg<1024, 64, 2, 2, 2, 16, 2, 2, true, false>>(L);
      if (L.K > 4096) return launch_logits_c<SplitCfg<1024, 128, 2, 2, 2, 8, 4, 1, true, false>>(L);
      return launch_logits_c<SplitCfg<1024, 128, 2, 2, 2, 16, 3, 1, true, false>, 3>(L);
    default: return hipErrorInvalidValue;
  }
}

// Reads L.logits as stored (L.logit_bf16 says which dtype).
hipError_t launch_route_select(const RouteLaunch &L) {
  switch (L.E) {
    case 64: return launch_select_e<64>(L);
    case 128: return launch_select_e<128>(L);
    case 256: return launch_select_e<256>(L);
    case 512: return launch_select_e<512>(L);
    case 1024: return launch_select_e<1024>(L);
    default: return hipErrorInvalidValue;
  }
}

bool fused_supports(int64_t E, int64_t K, bool x_f32) {
  return E == 256 && K >= 1 && K <= (x_f32 ? 16384 : 4096) && (K % (x_f32 ? 4 : 8)) == 0;
}

hipError_t launch_route_fused(const RouteLaunch &L) {
  if (L.E != 256) return hipErrorInvalidValue;
  if (!L.xf) return launch_logits_c<SplitCfg<256, 256, 2, 2, 1, 8, 4, 1, true, true>>(L);
  return launch_logits_c<SplitCfg<256, 256, 2, 2, 1, 8, 4, 1, true, false>>(L);
}

hipError_t launch_route_split(const RouteLaunch &L) {
  const hipError_t e = launch_route_logits(L);
  if (e != hipSuccess) return e;
  return launch_route_select(L);
}

}  // namespace drk
