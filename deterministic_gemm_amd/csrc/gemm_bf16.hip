// gemm_bf16.hip -- batch-invariant dense GEMM on bf16 matrix cores.
//
// out[M,N] = x[M,K] . W[K,N], bf16 inputs, fp32 accumulation.  A batch-
// invariant kernel must reduce K in one static order whatever the shape ("The
// Illusion of Determinism in Disaggregated Inference", section "The arithmetic
// cost of batch-invariant kernels").  Every output here is accumulated by the
// same instruction sequence: one v_mfma_f32_16x16x32_bf16 per 32-wide K step,
// k ascending, into one accumulator that starts at zero, with no split of K.
// The tile over M and N only decides which lanes run that sequence, so a row
// gets the same bits at every M, at every position in a tile and under every
// tile configuration.  The matrix core's internal order of the 32 products of
// one step is the hardware's; results are therefore compared with the exact
// product within a tolerance, and with themselves across M bit for bit.
//
// Data movement: x and W tiles go from global memory straight into LDS
// (16 bytes per lane, the LDS side written in order) through a ring of S
// stages of BK steps of K.  The x operand of a 16x16x32 step is eight
// consecutive k of one row: one 16-byte LDS read from x stored as [row][k],
// its 16-byte units XOR-swizzled by row so that one instruction's reads
// spread over the banks.  The W operand is eight consecutive k of one column,
// which W's [k][n] layout keeps 2N bytes apart, so it is read with the LDS
// transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element i % 4 of the 8 bytes read by lane i / 4 + 4j, j = 0..3.
// With lane i/4 + 4j reading row k0 + j at columns c0 + 4(i/4) .. +3, lane i
// gets column c0 + i at rows k0 .. k0+3; two such reads give the eight k.
// Tiles of 128 columns or more keep W in LDS in 128-byte blocks of four K rows
// by 16 columns, so each 16-lane group of a transpose read takes one whole
// 128-byte block instead of four 32-byte pieces of rows 2N bytes apart (the
// GEMM gained 1-5% at M = 512-4096, K = N = 4096).  Each transfer lane
// fetches the 16-byte unit that its LDS position holds, so global reads stay
// runs of 256 bytes per row.  Narrower tiles keep [k][n] rows with
// XOR-swizzled units.
#include <type_traits>
#include <utility>

#include "lds_dma.h"
#include "buf_dma.h"
#include "launch.h"

namespace drk {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, each i a constant
// expression inside f.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

static __device__ const Pad16 g_zero16 = {{0.0f, 0.0f, 0.0f, 0.0f}};

template <int BM_, int BN_, int WM_, int WN_, int BK_, int S_, bool ROT_ = false>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, S = S_;
  static constexpr bool ROT = ROT_;  // the rotated loop (gemm_tile_rot)
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;  // rows, columns per wavefront
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 tiles per wavefront
  static constexpr int UA = BK / 8;                 // 16-byte units per x row of a stage
  static constexpr int UB = BN / 8;                 // 16-byte units per W row of a stage
  static constexpr int NB = BN / 16;                // W blocks of 16 columns
  static constexpr int AU = BM * UA, BU = BK * UB;  // units per stage
  static constexpr int ABYTES = AU * 16, STAGE = (AU + BU) * 16;
  static constexpr int PER = (AU + BU) / 64 / NW;   // transfers per wavefront per stage
  static_assert(FM >= 1 && FN >= 1 && TM * WM == BM && TN * WN == BN, "wavefront tiles");
  static_assert(BK % 32 == 0 && (UA == 4 || UA == 8 || UA == 16 || UA == 32), "K steps per stage");
  static_assert(NB % 2 == 0 && (BN >= 128 || UB == 4 || UB == 8), "W layout");
  static_assert(AU % 64 == 0 && BU % 64 == 0 && PER * 64 * NW == AU + BU, "transfers split evenly");
  static_assert(PER * (S - 1) <= 63 && S >= 2, "vmcnt range");
  static_assert(S * STAGE <= 160 * 1024, "LDS");
  // x rows: unit u of row r sits at u ^ swa(r); 16 consecutive rows reading
  // the same unit then hit 16 distinct 16-byte bank groups.
  __host__ __device__ static constexpr int swa(int r) { return UA >= 16 ? r % 16 : (r / (16 / UA)) % UA; }
  // W, tiles of 128 columns or more (QB): rows 4q .. 4q+3 by columns
  // 16b .. 16b+15 form a 128-byte block, row-major, at block
  // q * NB + (b ^ ((q >> 1) & 1)).  The xor puts the blocks that groups g
  // and g+1 of one read take (q two apart) on alternate 128-byte halves of
  // each 256 bytes, as a contiguous 512-byte read would be.  Narrower tiles keep W
  // row-major ([k][n], unit u of row k at u ^ swb(k)): their transfers then
  // read whole 64- or 128-byte row pieces with consecutive lanes, where the
  // blocks would alternate rows every two lanes (measured 7% slower at
  // M = 128, K = N = 4096).
  static constexpr bool QB = BN >= 128;
  __host__ __device__ static constexpr int swb(int k) {
    return UB == 8 ? ((k % 4) >> 1) + 2 * ((k / 8) % 4) : (k / 8) % 4;
  }
  // Unit p of the stage's W part holds row kr, columns nc .. nc+7.
  __host__ __device__ static constexpr void b_unit(int p, int &kr, int &nc) {
    if (QB) {
      const int q = p / (BN / 2), r = p % (BN / 2);
      kr = 4 * q + (r % 8) / 2;
      nc = 16 * ((r / 8) ^ ((q >> 1) & 1)) + 8 * (r % 2);
    } else {
      kr = p / UB;
      nc = 8 * ((p % UB) ^ swb(kr));
    }
  }
  // Byte offset of what lane (g4, tj, tq) of a transpose read takes for K
  // step kk, half c (rows 4c .. 4c+3 of its group of 8) and column fragment
  // b: row kk*32 + 8 g4 + 4 c + tj, columns 16 b + 4 tq .. +3.
  __host__ __device__ static constexpr int b_off(int kk, int g4, int c, int tj, int tq, int b) {
    if (QB) {
      const int q = 8 * kk + 2 * g4 + c;
      return (q * NB + (b ^ (g4 & 1))) * 128 + tj * 32 + tq * 8;
    }
    const int kr = kk * 32 + 8 * g4 + 4 * c + tj, col = b * 16 + 4 * tq;
    return (kr * UB + ((col / 8) ^ swb(kr))) * 16 + (col % 8) * 2;
  }
};

// Source row of each of this lane's x transfers (the same rows every stage):
// tile row r -> output row m0 + r, read from x row rows[m0 + r] (or m0 + r),
// or -1 past the tile's last row [mend) or for a source outside [0, Mx).
template <class C>
__device__ __forceinline__ void gemm_arows(const int32_t *__restrict__ rows, int64_t Mx, int64_t m0, int64_t mend,
                                           int wave, int lane, int32_t (&arow)[C::PER]) {
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int p = (wave * C::PER + i) * 64 + lane;
    arow[i] = -1;
    if (p < C::AU) {
      const int64_t g = m0 + p / C::UA;
      if (g < mend) {
        const int64_t r = rows ? rows[g] : g;
        arow[i] = (r >= 0 && r < Mx) ? static_cast<int32_t>(r) : -1;
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void gemm_issue(const uint16_t *__restrict__ x, const int32_t (&arow)[C::PER],
                                           const uint16_t *__restrict__ W, int K, int N, int n0, int st, int nst,
                                           int wave, int lane, char *stage) {
  const int k0 = st * C::BK;
  const bool live = st < nst;
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int p = (wave * C::PER + i) * 64 + lane;  // unit within the stage
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage + (wave * C::PER + i) * 1024)));
    const void *src = &g_zero16;
    if (p < C::AU) {
      const int r = p / C::UA, up = p % C::UA;
      const int u = up ^ C::swa(r);
      const int k = k0 + 8 * u;
      if (live && arow[i] >= 0 && k < K) src = x + static_cast<int64_t>(arow[i]) * K + k;
    } else {
      int kr = 0, nc = 0;
      C::b_unit(p - C::AU, kr, nc);
      const int k = k0 + kr;
      if (live && k < K) src = W + static_cast<int64_t>(k) * N + n0 + nc;
    }
    dma16(src, lds);
  }
}

// The same transfers through buffer descriptors (the path for operands under
// 4 GiB).  A lane keeps one 32-bit byte offset per transfer for the whole
// tile; each stage moves the descriptors' bases (scalar work) to K-step k0 and
// shrinks their ranges to what is left of the operand.  A transfer whose
// offset lies past the range reads zeros without touching memory (checked
// per 4-byte word), which covers rows that read a zero row, W rows past K and
// stages past the last; x units past K in a partial stage read the next row's
// data, which no matrix step consumes.  Fewer registers than 64-bit
// addresses, so deeper rings fit a wavefront's budget.
template <class C>
__device__ __forceinline__ void gemm_voffs(const int32_t (&arow)[C::PER], int K, int N, int n0, int wave, int lane,
                                           uint32_t (&voff)[C::PER]) {
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int p = (wave * C::PER + i) * 64 + lane;
    if (p < C::AU) {
      const int r = p / C::UA, up = p % C::UA;
      const int u = up ^ C::swa(r);
      voff[i] = arow[i] >= 0 ? static_cast<uint32_t>((static_cast<int64_t>(arow[i]) * K + 8 * u) * 2) : kBufFarOff;
    } else {
      int kr = 0, nc = 0;
      C::b_unit(p - C::AU, kr, nc);
      voff[i] = static_cast<uint32_t>((static_cast<int64_t>(kr) * N + n0 + nc) * 2);
    }
  }
}

template <class C>
__device__ __forceinline__ void gemm_issue_buf(const uint16_t *__restrict__ x, int64_t Mx,
                                               const uint16_t *__restrict__ W, int K, int N,
                                               const uint32_t (&voff)[C::PER], int st, int nst, int wave,
                                               char *stage) {
  const int64_t k0 = static_cast<int64_t>(st) * C::BK;
  const bool live = st < nst;
  const u32x4 xr = buf_rsrc(x + k0, live ? (Mx * K - k0) * 2 : 0);
  const u32x4 wr = buf_rsrc(W + k0 * N, live ? (K - k0) * static_cast<int64_t>(N) * 2 : 0);
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage + (wave * C::PER + i) * 1024)));
    // a transfer is all x or all W (AU is a multiple of 64)
    dma16_buf(voff[i], (wave * C::PER + i) * 64 < C::AU ? xr : wr, lds);
  }
}

// Round to nearest even on the 16 dropped bits (NaN -> 0x7FC0).
__device__ __forceinline__ uint16_t gemm_f32_to_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One 32-wide K step of a wavefront's tile from the stage at As (x) / Bs (W).
template <class C>
__device__ __forceinline__ void gemm_kstep(const char *As, const char *Bs, int kk, int wm, int wn, int r16, int g4,
                                           int tj, int tq, f32x4 (&acc)[C::FM][C::FN]) {
  constexpr int FM = C::FM, FN = C::FN;
  bf16x8 af[FM], bfv[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * C::TM + i * 16 + r16;
    const int u = (kk * 4 + g4) ^ C::swa(r);
    af[i] = *reinterpret_cast<const bf16x8 *>(As + (r * C::UA + u) * 16);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    i16x4 h[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const char *a = Bs + C::b_off(kk, g4, c, tj, tq, wn * FN + j);
      h[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(a));
    }
    const i16x4 lo = h[0], hi = h[1];
    bfv[j] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                            lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
}

// One whole stage (BK / 32 K steps) of a wavefront's tile, with the operand
// reads running ahead of the matrix steps: the x fragment of step t + AD (a
// step is one K step of one 16-row fragment) and the W fragments of the next
// K step are read from LDS while the matrix steps of step t run, into a ring
// of AD + 1 x fragments and two sets of W fragments, each read issued between
// two matrix steps.  The same instructions and operands per output as
// gemm_kstep, in the same order per accumulator, so the bits are the same.
template <class C>
__device__ __forceinline__ void gemm_stage_pipelined(const char *As, const char *Bs, int wm, int wn, int r16, int g4,
                                                     int tj, int tq, f32x4 (&acc)[C::FM][C::FN]) {
  constexpr int FM = C::FM, FN = C::FN, KK = C::BK / 32, T = KK * FM;
  constexpr int BSTEP = FM > 1 ? FM / 2 : 0;  // the step of each K step that reads the next W fragments
  constexpr int AD = 2;  // x fragments read ahead
  bf16x8 af[AD + 1], bfv[2][FN];
  const auto read_a = [&](int t, bf16x8 &dst) {
    const int kk = t / FM, i = t % FM;
    const int r = wm * C::TM + i * 16 + r16;
    const int u = (kk * 4 + g4) ^ C::swa(r);
    dst = *reinterpret_cast<const bf16x8 *>(As + (r * C::UA + u) * 16);
  };
  const auto read_b = [&](int kk, bf16x8 (&dst)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      i16x4 h[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const char *a = Bs + C::b_off(kk, g4, c, tj, tq, wn * FN + j);
        h[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(a));
      }
      const i16x4 lo = h[0], hi = h[1];
      dst[j] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                              lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
  };
  read_b(0, bfv[0]);
  static_for<AD>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    if constexpr (t < T) read_a(t, af[t]);
  });
  static_for<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    constexpr int kk = t / FM, i = t % FM;
    constexpr bool ra = t + AD < T, rb = i == BSTEP && kk + 1 < KK;
    constexpr int nr = (ra ? 1 : 0) + (rb ? 2 * FN : 0);  // LDS reads issued in this step
    if constexpr (ra) read_a(t + AD, af[(t + AD) % (AD + 1)]);
    if constexpr (rb) read_b(kk + 1, bfv[(kk + 1) % 2]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t % (AD + 1)], bfv[kk % 2][j], acc[i][j], 0, 0, 0);
    // one read after each matrix step, the rest after the step's last one
    constexpr int inter = nr < FN ? nr : FN;
    static_for<inter>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
    if constexpr (FN > inter) __builtin_amdgcn_sched_group_barrier(0x008, FN - inter, 0);
    if constexpr (nr > inter) __builtin_amdgcn_sched_group_barrier(0x100, nr - inter, 0);
  });
}

// Stores a wavefront's tile: rows [m0, mend) only, fp32 or rounded to bf16.
template <class C, class OutT>
__device__ __forceinline__ void gemm_store(const f32x4 (&acc)[C::FM][C::FN], OutT *__restrict__ out, int64_t m0,
                                           int64_t mend, int N, int n0, int wm, int wn, int r16, int g4) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = m0 + wm * C::TM + i * 16 + g4 * 4 + q;
      if (m >= mend) continue;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if constexpr (sizeof(OutT) == 2) out[m * N + n0 + wn * C::TN + j * 16 + r16] = gemm_f32_to_bf16(acc[i][j][q]);
        else out[m * N + n0 + wn * C::TN + j * 16 + r16] = acc[i][j][q];
      }
    }
}

// The rotated loop, for stages of KK = BK / 32 K steps (one or two) in a
// ring of S stages, W in 128-byte blocks and an even number of column
// fragments.  The plain loop reads a stage's fragments right after its
// barrier, so every wavefront of the workgroup reads at once while the
// matrix cores idle.  Here step t's matrix instructions run on fragments
// already in registers, and step t+1's fragments are read between them: x
// fragment i right after the FN matrix steps that use fragment i (into the
// same registers), the W fragments of step t+1 into a second set over the
// first FN/2 rows.  When step t+1 lies in the next stage, step t first
// waits for its own reads of the current stage (lgkmcnt) and for the next
// stage's transfers (vmcnt); the barrier then makes the next stage visible
// and frees the current stage's buffer, which takes stage s+S's transfers at
// once.  Two-step stages read x in 128-byte row pieces, which the L2s serve
// at a higher rate than 64-byte ones (the operand transfers of a 256 x 256
// tile over K = 4096 alone: 57 against 75 us).  The same instructions and
// operands per output as gemm_kstep, in the same order per accumulator, so
// the bits are the same.
template <class C, class OutT, bool SKIP, bool BUF>
__device__ __forceinline__ void gemm_tile_rot(const uint16_t *__restrict__ x, const int32_t *__restrict__ rows,
                                              int64_t Mx, const uint16_t *__restrict__ W, OutT *__restrict__ out,
                                              int64_t m0, int64_t mend, int K, int N, int n0, char *smem) {
  constexpr int FM = C::FM, FN = C::FN, S = C::S, KK = C::BK / 32;
  static_assert((KK == 1 || KK == 2) && S >= 3 - (KK - 1) && C::QB && FN % 2 == 0 && FN / 2 <= FM,
                "rotated loop");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int ta = lane & 15, tj = ta >> 2, tq = ta & 3;
  const int nk = K / 32;              // K steps
  const int nst = (nk + KK - 1) / KK;  // stages
  const bool wlive =
      !SKIP || __builtin_amdgcn_readfirstlane(static_cast<int>(m0 + static_cast<int64_t>(wm) * C::TM < mend)) != 0;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  int32_t arow[C::PER];
  gemm_arows<C>(rows, Mx, m0, mend, wave, lane, arow);
  uint32_t voff[C::PER];
  if constexpr (BUF) gemm_voffs<C>(arow, K, N, n0, wave, lane, voff);
  const auto issue = [&](int st) {
    char *stage = smem + (st % S) * C::STAGE;
    if constexpr (BUF) gemm_issue_buf<C>(x, Mx, W, K, N, voff, st, nst, wave, stage);
    else gemm_issue<C>(x, arow, W, K, N, n0, st, nst, wave, lane, stage);
  };

  // Per-lane byte offsets within a stage.  x fragment i of this wavefront at
  // step kk of the stage is row wm*TM + 16i + r16, unit (4 kk + g4) ^
  // swa(row); swa repeats every 16 rows, so fragment i sits i * 16 UA * 16
  // bytes after fragment 0.  W fragment j of half c at step kk is block
  // (8 kk + 2 g4 + c) * NB + ((wn*FN + j) ^ s), s = g4 & 1: even j at
  // boff0 + 128 j, odd j at boff1 + 128 j.
  static_assert((C::UA == 4 || C::UA == 8) && C::swa(16) == C::swa(0), "x fragments 16 rows apart");
  const int arow0 = wm * C::TM + r16;
  int aoff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) aoff[kk] = (arow0 * C::UA + ((4 * kk + g4) ^ C::swa(arow0))) * 16;
  const int s1 = g4 & 1;
  const int bbase = ((2 * g4) * C::NB + wn * FN) * 128 + tj * 32 + tq * 8;
  const int boff0 = bbase + s1 * 128, boff1 = bbase - s1 * 128;
  const auto read_a = [&](const char *st, int kk, int i) {
    return *reinterpret_cast<const bf16x8 *>(st + aoff[kk] + i * 16 * C::UA * 16);
  };
  const auto read_bh = [&](const char *st, int kk, int j, int c) {
    const char *a = st + C::ABYTES + ((j & 1) ? boff1 : boff0) + j * 128 + (8 * kk + c) * C::NB * 128;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(a));
  };
  const auto join = [](i16x4 lo, i16x4 hi) {
    return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0],
                                                                                    hi[1], hi[2], hi[3]});
  };

  bf16x8 af[FM], b0[FN], b1[FN];
  // matrix steps of one K step on af / bc, reading the next step's fragments
  // (step kn of stage buffer nx) between them
  const auto mstep = [&](bf16x8(&bc)[FN], bf16x8(&bn)[FN], const char *nx, int kn) {
    i16x4 bh[FN][2];
    static_for<FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      // rows 0 .. FN/2 - 1 read four W halves each (two fragments), the rest none
      constexpr int nb = i < FN / 2 ? 4 : 0;
      static_for<FN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bc[j], acc[i][j], 0, 0, 0);
      });
      if constexpr (nb > 0) {
        static_for<2>([&](auto jc) {
          constexpr int j = 2 * i + decltype(jc)::value;
          bh[j][0] = read_bh(nx, kn, j, 0);
          bh[j][1] = read_bh(nx, kn, j, 1);
          bn[j] = join(bh[j][0], bh[j][1]);
        });
      }
      af[i] = read_a(nx, kn, i);
      // one LDS read after each of the row's first matrix steps, the rest after
      constexpr int nr = nb + 1;
      constexpr int inter = nr < FN ? nr : FN;
      static_for<inter>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
      if constexpr (FN > inter) __builtin_amdgcn_sched_group_barrier(0x008, FN - inter, 0);
      if constexpr (nr > inter) __builtin_amdgcn_sched_group_barrier(0x100, nr - inter, 0);
      // nothing crosses a row: a new x fragment is never read while the
      // old one still waits for its matrix steps
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  const auto read_first = [&]() {
    if (!SKIP || wlive) {
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = read_a(smem, 0, i);
#pragma unroll
      for (int j = 0; j < FN; ++j) b0[j] = join(read_bh(smem, 0, j, 0), read_bh(smem, 0, j, 1));
    }
  };
  // this wavefront's LDS reads done, then the barrier
  const auto sync = [&]() {
    compiler_fence();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };
  // At the last step of stage s: wait for stage s+1 and this wavefront's
  // reads of stage s, make stage s+1 visible and stage s's buffer free,
  // refill it with stage s+S.  The last step also reads "step nk" (of the
  // last stage, or of stage nst, issued as zeros and waited for like any
  // other); its fragments go unused, so there is one loop body and no tail
  // copy.
#pragma unroll
  for (int i = 0; i < S; ++i) issue(i);
  compiler_fence();
  wait_vmcnt<C::PER * (S - 1)>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  read_first();
  for (int s = 0; s < nst; ++s) {
    static_for<KK>([&](auto kc) {
      constexpr int kk = decltype(kc)::value;
      const int t = s * KK + kk;
      if (t < nk) {
        if constexpr (kk == KK - 1) {
          compiler_fence();
          wait_vmcnt<C::PER * (S - 2)>();
          sync();
          issue(s + S);
        }
        if (!SKIP || wlive) {
          if constexpr (kk == KK - 1) mstep(b0, b1, smem + ((s + 1) % S) * C::STAGE, 0);
          else mstep(b0, b1, smem + (s % S) * C::STAGE, kk + 1);
#pragma unroll
          for (int j = 0; j < FN; ++j) b0[j] = b1[j];
        }
      }
    });
  }
  // no transfer may still be writing this workgroup's LDS when it moves on
  compiler_fence();
  wait_vmcnt<0>();
  gemm_store<C>(acc, out, m0, mend, N, n0, wm, wn, r16, g4);
}

// One output tile: rows [m0, min(m0 + BM, mend)) and columns [n0, n0 + BN) of
// out = x[rows] . W, every output reduced by the same instruction sequence;
// stored as fp32, or rounded to bf16 (OutT = uint16_t).  With SKIP, a
// wavefront whose rows all lie past the tile's last row (in a ragged grouped
// tile) skips its LDS reads and matrix steps but still moves its share of the
// transfers and meets every barrier; the dense kernel, whose only partial
// tile is the last, measured faster without the branch.
template <class C, class OutT = float, bool SKIP = false, bool BUF = false>
__device__ __forceinline__ void gemm_tile(const uint16_t *__restrict__ x, const int32_t *__restrict__ rows,
                                          int64_t Mx, const uint16_t *__restrict__ W, OutT *__restrict__ out,
                                          int64_t m0, int64_t mend, int K, int N, int n0, char *smem) {
  if constexpr (C::ROT) {
    gemm_tile_rot<C, OutT, SKIP, BUF>(x, rows, Mx, W, out, m0, mend, K, N, n0, smem);
    return;
  }
  constexpr int FM = C::FM, FN = C::FN, S = C::S;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int nst = (K + C::BK - 1) / C::BK;
  const bool wlive =
      !SKIP || __builtin_amdgcn_readfirstlane(static_cast<int>(m0 + static_cast<int64_t>(wm) * C::TM < mend)) != 0;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // per-lane parts of the operand addresses
  const int ta = lane & 15;          // transpose read: source lane within its group
  const int tj = ta >> 2, tq = ta & 3;
  int32_t arow[C::PER];
  gemm_arows<C>(rows, Mx, m0, mend, wave, lane, arow);
  uint32_t voff[C::PER];
  if constexpr (BUF) gemm_voffs<C>(arow, K, N, n0, wave, lane, voff);
  const auto issue = [&](int st) {
    char *stage = smem + (st % S) * C::STAGE;
    if constexpr (BUF) gemm_issue_buf<C>(x, Mx, W, K, N, voff, st, nst, wave, stage);
    else gemm_issue<C>(x, arow, W, K, N, n0, st, nst, wave, lane, stage);
  };

#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(i);

  for (int st = 0; st < nst; ++st) {
    compiler_fence();
    wait_vmcnt<C::PER * (S - 2)>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    issue(st + S - 1);
    const char *As = smem + (st % S) * C::STAGE;
    const char *Bs = As + C::ABYTES;
    const int nsub = (K - st * C::BK) < C::BK ? (K - st * C::BK) / 32 : C::BK / 32;
    if (!SKIP || wlive) {
      // wavefront tiles of up to 8 fragments: the larger ones (64 x 64 and
      // 128 x 64) measured slower pipelined (86 against 77 us at M = 2048,
      // K = N = 4096) or ran out of registers
      bool done = false;
      if constexpr (C::FM * C::FN <= 8) {
        if (nsub == C::BK / 32) {
          gemm_stage_pipelined<C>(As, Bs, wm, wn, r16, g4, tj, tq, acc);
          done = true;
        }
      }
      if (!done) {
#pragma unroll
        for (int kk = 0; kk < C::BK / 32; ++kk)
          if (kk < nsub) gemm_kstep<C>(As, Bs, kk, wm, wn, r16, g4, tj, tq, acc);
      }
    }
  }
  // no transfer may still be writing this workgroup's LDS when it moves on
  compiler_fence();
  wait_vmcnt<0>();
  gemm_store<C>(acc, out, m0, mend, N, n0, wm, wn, r16, g4);
}

// Workgroups go to the eight XCDs in turn (linear index L to XCD L % 8).
// With gy > 0 the tile grid is cut into gy x (8 / gy) rectangles and XCD j
// takes rectangle j: its L2 then reads x for the rectangle's row tiles and W
// for its column tiles only (at 16 x 16 tiles, 24 of 64 MiB instead of all of
// x and an eighth of W).  Otherwise, with a multiple of eight column tiles,
// XCD j takes the j-th contiguous eighth of them with every row tile, so
// neighbouring tiles that share 128-byte lines of W read them through one L2.
template <class C, class OutT, bool BUF>
__global__ __launch_bounds__(C::NT) void gemm_bf16_kernel(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ W,
                                                         OutT *__restrict__ out, int64_t M, int K,
                                                         int N, int gy) {
  __shared__ __attribute__((aligned(16))) char smem[C::S * C::STAGE];
  const int nx = gridDim.x, ny = gridDim.y;
  int bx, by;
  if (gy > 0) {
    const int L = blockIdx.x + blockIdx.y * nx;
    const int xcd = L % 8, slot = L / 8;
    const int gx = 8 / gy, rb = ny / gy, cb = nx / gx;  // tiles per rectangle: rb x cb
    by = (xcd / gx) * rb + slot / cb;
    bx = (xcd % gx) * cb + slot % cb;
  } else {
    by = blockIdx.y;
    bx = (nx % 8 == 0) ? (blockIdx.x % 8) * (nx / 8) + blockIdx.x / 8 : blockIdx.x;
  }
  gemm_tile<C, OutT, false, BUF>(x, nullptr, M, W, out, static_cast<int64_t>(by) * C::BM, M, K, N, bx * C::BN,
                                 smem);
}

// Grouped (per-expert) product: expert e owns output rows [offsets[e],
// offsets[e+1]) and multiplies them by W[e].  Row tiles never straddle two
// experts: expert e has ceil(count_e / BM) of them -- or one of the taller
// tile when BM < count_e <= its height (+ GG_TAIL rows, taken by a second
// pass), which streams W[e]'s column strip once where a full and a ragged tile
// would stream it twice -- numbered after those of
// experts < e, T in all; a workgroup finds the expert of its row tile by a
// scan of the tile counts in LDS.  Workgroups go to the eight XCDs in turn
// (linear index L to XCD L % 8); XCD c takes the c-th contiguous eighth of
// the T row tiles with all their column tiles, one row tile's columns after
// another.  So an expert's rows and weights are read into one XCD's L2 (a
// column-major order makes every XCD read all of x).  The grid is sized for
// the most row tiles any routing can give; workgroups past the last tile of
// their XCD's share exit.  Every output row is reduced by the dense kernel's
// instruction sequence, so a row has the same bits whatever its group's size
// or position, and the same bits as dr_gemm_bf16 of that row with W[e].
constexpr int GG_EMAX = 1024;
// An expert of up to this many rows past the taller tile's height takes the
// taller tile and, in the same workgroup, a second pass over its last rows
// (which streams the expert's weight strip again), instead of a second row
// tile: with row tiles a multiple of the CUs, one more row tile is one more
// round of workgroups.
constexpr int GG_TAIL = 64;

template <class C, class CT, bool BUF>
__global__ __launch_bounds__(C::NT) void grouped_gemm_bf16_kernel(const uint16_t *__restrict__ x, int64_t Mx,
                                                                 const int32_t *__restrict__ rows,
                                                                 const uint16_t *__restrict__ W,
                                                                 const int32_t *__restrict__ offsets, int E,
                                                                 int64_t P, float *__restrict__ out, int K, int N,
                                                                 int ncol) {
  constexpr int EPL = (GG_EMAX + C::NT - 1) / C::NT;  // experts per lane in the scan
  // CT: the taller tile, for an expert of more than C::BM and at most CT::BM
  // rows (CT = C: none)
  constexpr bool TALL = CT::BM > C::BM;
  static_assert(CT::NT == C::NT && CT::BN == C::BN && CT::BM >= C::BM, "tile pair");
  constexpr int SMEM = C::S * C::STAGE > CT::S * CT::STAGE ? C::S * C::STAGE : CT::S * CT::STAGE;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ int32_t tstart[GG_EMAX + 1];
  __shared__ int32_t wsum[C::NW];
  __shared__ int32_t found;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // row tiles of lane t's experts EPL*t .. EPL*t + EPL - 1, and their scan
  int cnt[EPL], v = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = EPL * t + i;
    const int c = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    cnt[i] = (TALL && c > C::BM && c <= CT::BM + GG_TAIL) ? 1 : (c + C::BM - 1) / C::BM;
    v += cnt[i];
  }
  const int mine = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  if (t == 0) found = -1;
  __syncthreads();
  int start = v - mine, total = 0;
  for (int w = 0; w < C::NW; ++w) {
    if (w < wave) start += wsum[w];
    total += wsum[w];
  }
  // this workgroup's row tile and column tile
  const int xcd = static_cast<int>(blockIdx.x % 8), slot = static_cast<int>(blockIdx.x / 8);
  const int share = (total + 7) / 8;  // row tiles per XCD
  const int tr = slot / ncol;
  const int tile = (tr < share) ? xcd * share + tr : 0x7FFFFFFF;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = EPL * t + i;
    if (e < E) {
      if (tile >= start && tile < start + cnt[i]) found = e;
      tstart[e] = start;
    }
    start += cnt[i];
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(found);
  if (e < 0) return;  // past the last tile (uniform over the workgroup)
  const int64_t lo = offsets[e], mend = offsets[e + 1];
  if (lo < 0 || mend > P || mend < lo) return;  // inconsistent offsets: nothing is written outside out
  const int64_t m0 = lo + static_cast<int64_t>(tile - tstart[e]) * C::BM;
  const uint16_t *We = W + static_cast<int64_t>(e) * K * N;
  const int n0 = (slot % ncol) * C::BN;
  if (TALL && mend - lo > C::BM && mend - lo <= CT::BM + GG_TAIL) {
    const int64_t mt = mend - lo <= CT::BM ? mend : lo + CT::BM;
    gemm_tile<CT, float, true, BUF>(x, rows, Mx, We, out, lo, mt, K, N, n0, smem);
    if (mt < mend) {
      // the last rows, at most GG_TAIL (one wavefront band of the smaller
      // tile holds them; the other skips): every wavefront is done with the
      // LDS stages before the second pass refills them
      __syncthreads();
      gemm_tile<C, float, true, BUF>(x, rows, Mx, We, out, mt, mend, K, N, n0, smem);
    }
  } else {
    gemm_tile<C, float, true, BUF>(x, rows, Mx, We, out, m0, mend, K, N, n0, smem);
  }
}

// Small batches (M <= 128): one workgroup per 16-column strip of W, holding
// every row of the batch.  At these sizes W (32 MiB at K = N = 4096) is read
// once and every CU also reads all of x (up to 1 MiB) from L2; each path
// needs many bytes in flight per CU, and one 16-row fragment's accumulator
// is a chain of K/32 dependent matrix steps.  The operands take separate
// routes.  NP producer wavefronts only move W into a deep LDS ring (S stages
// of BK K rows x 16 columns) and count their own transfers.  Each of the NC
// compute wavefronts owns one 16-row fragment of x: it loads the fragment
// into registers in chunks of four K steps, R - 1 chunks ahead, 256
// contiguous bytes per row per chunk (one row per 16 lanes, so each load
// touches few cache lines), writes each chunk into a private pair of LDS
// buffers, and reads the matrix core's A operand back from there.  Its loads
// are the compiler's, so keeping the two kinds of memory operation in
// different wavefronts keeps each wavefront's in-order wait counter exact
// for what it waits on.  The W stages are long (BK = 512) so that the
// workgroup meets at few barriers.  Each output is reduced by the dense
// kernel's instruction sequence -- one v_mfma_f32_16x16x32_bf16 per 32-wide
// K step, k ascending, one accumulator from zero, row r16 / column r16 and
// k = 32t + 8 g4 .. +7 in lane (g4, r16) -- so rows are bit-identical to
// every other tile configuration.
template <int NC_, int NP_, int S_, int R_>
struct StripCfg {
  static constexpr int NC = NC_, NP = NP_, S = S_, R = R_;
  static constexpr int BK = 512, KS = BK / 32;  // K rows, 32-wide K steps per W stage
  static constexpr int CH = 4;                  // K steps per x chunk
  static constexpr int CPS = KS / CH;           // x chunks per W stage
  static constexpr int NW = NC + NP, NT = 64 * NW;
  static constexpr int STAGE = BK * 32;    // bytes of W per stage: BK rows of 16 bf16
  static constexpr int DI = STAGE / 1024;  // transfers (64 lanes x 16 bytes) per stage
  static constexpr int PW = DI / NP;       // ... per producer wavefront
  static constexpr int XB = 16 * CH * 64;  // bytes of one x fragment per chunk
  static constexpr int XBASE = S * STAGE;  // compute wavefront w's buffers at XBASE + 2 XB w
  static constexpr int U = R > CPS ? R / CPS : 1;  // W stages per unrolled loop body
  static constexpr int LDS = XBASE + 2 * XB * NC;
  static_assert(NC >= 1 && NW <= 16, "wavefronts");
  static_assert(PW * NP == DI && PW >= 1, "transfers split evenly");
  static_assert(PW * (S - 2) <= 63 && S >= 3, "vmcnt range");
  static_assert(R >= 2 && (R % CPS == 0 || CPS % R == 0) && CPS % 2 == 0, "x ring: whole bodies");
  static_assert(LDS <= 160 * 1024, "LDS");
  // W in a stage: [k][16], 16-byte unit p (LDS byte 16 p) holds row p / 2,
  // columns nc .. nc+7; the two units of a row swap on alternate groups of 8
  // rows, so the transpose reads of one instruction spread over the banks.
  __host__ __device__ static constexpr void b_unit(int p, int &kr, int &nc) {
    kr = p / 2;
    nc = 8 * ((p % 2) ^ ((kr / 8) % 2));
  }
  // Byte offset of what lane (g4, tj, tq) of a transpose read takes for K
  // step kk of the stage, half c: row 32 kk + 8 g4 + 4 c + tj, columns 4 tq .. +3.
  __host__ __device__ static constexpr int b_off(int kk, int g4, int c, int tj, int tq) {
    const int kr = kk * 32 + 8 * g4 + 4 * c + tj, col = 4 * tq;
    return (kr * 2 + ((col / 8) ^ ((kr / 8) % 2))) * 16 + (col % 8) * 2;
  }
};

template <class C, class OutT>
__global__ __launch_bounds__(C::NT) void gemm_strip_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ W,
                                                          OutT *__restrict__ out, int M, int K, int N) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  // XCD j takes the j-th contiguous eighth of the strips, so the four strips
  // of a 128-byte line of W read it through one L2
  const int nx = gridDim.x;
  const int bx = (nx % 8 == 0) ? (blockIdx.x % 8) * (nx / 8) + blockIdx.x / 8 : blockIdx.x;
  const int n0 = bx * 16;
  constexpr int S = C::S, KS = C::KS, CH = C::CH, CPS = C::CPS, U = C::U, R = C::R;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nk = K / 32;               // K steps
  const int nst = (nk + KS - 1) / KS;  // W stages
  const int nch = (nk + CH - 1) / CH;  // x chunks

  if (wave >= C::NC) {
    // producer: W stages into the ring, S - 1 ahead of the compute wavefronts.
    // Stages past the last read zeros through an empty range, so every stage
    // issues the same number of transfers and the wait below stays exact.
    const int p = wave - C::NC;
    uint32_t voff[C::PW];
#pragma unroll
    for (int i = 0; i < C::PW; ++i) {
      int kr = 0, nc = 0;
      C::b_unit((p * C::PW + i) * 64 + lane, kr, nc);
      voff[i] = static_cast<uint32_t>((static_cast<int64_t>(kr) * N + n0 + nc) * 2);
    }
    const auto issue = [&](int st) {
      const int64_t k0 = static_cast<int64_t>(st) * C::BK;
      const u32x4 wr = buf_rsrc(W + k0 * N, st < nst ? (K - k0) * static_cast<int64_t>(N) * 2 : 0);
      char *stage = smem + (st % S) * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::PW; ++i) {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage + (p * C::PW + i) * 1024)));
        dma16_buf(voff[i], wr, lds);
      }
    };
#pragma unroll
    for (int i = 0; i < S - 1; ++i) issue(i);
    for (int st = 0; st < nst; ++st) {
      // this wavefront's transfers of stage st are done; after the barrier
      // all are, and stage st - 1's buffer has been read by everyone
      compiler_fence();
      wait_vmcnt<C::PW * (S - 2)>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      issue(st + S - 1);
    }
    // no transfer may still be writing this workgroup's LDS when it ends
    compiler_fence();
    wait_vmcnt<0>();
    return;
  }

  // compute wavefront `wave`: rows 16 wave .. +15; rows past M read zeros
  // through the range of x's descriptor and are not stored.  Loads past the
  // last K step read the next row's data or zeros and are never consumed, so
  // whole loop bodies carry no per-step branch (the compiler's waits on the
  // loads stay counts, not full drains); a ragged remainder runs the same
  // body with guards.
  const int r16 = lane & 15, g4 = lane >> 4;
  const int ta = lane & 15, tj = ta >> 2, tq = ta & 3;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x), static_cast<short>(0), M * K * 2, 0x00020000);
  // load j (0..3) of a chunk: row 4j + lane / 16, bytes 16 (lane % 16) of the
  // row's 256 for the chunk; written to the fragment buffer [16 rows][16
  // units] with unit u of row r at u ^ r (the writes and the A reads below
  // then take distinct banks within each 16 lanes)
  const int lr = lane >> 4, lu = lane & 15;
  uint32_t xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = wave * 16 + 4 * j + lr;
    xoff[j] = static_cast<uint32_t>(row < M ? (row * K + 8 * lu) * 2 : 0x7FFFFFF0);
  }
  char *xl = smem + C::XBASE + wave * 2 * C::XB;
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 xg[R][4];
  const auto load_chunk = [&](int c, u4(&dst)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[j] + c * 256, 0, 0);
  };
  const auto write_chunk = [&](const u4(&src)[4], int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * j + lr;
      *reinterpret_cast<u4 *>(xl + buf * C::XB + r * 256 + ((lu ^ r) * 16)) = src[j];
    }
  };
  bf16x8 af[CH];
  const auto read_a = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < CH; ++kk)
      af[kk] = *reinterpret_cast<const bf16x8 *>(xl + buf * C::XB + r16 * 256 + (((kk * 4 + g4) ^ r16) * 16));
  };
  const auto read_b = [&](const char *Bs, int kk) {
    i16x4 h[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
      h[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(Bs + C::b_off(kk, g4, c, tj, tq)));
    return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){h[0][0], h[0][1], h[0][2], h[0][3],
                                                                                  h[1][0], h[1][1], h[1][2], h[1][3]});
  };
  const auto sync = [&]() {
    // this wavefront's LDS reads so far are done before the barrier lets a
    // producer refill a stage buffer they read
    compiler_fence();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };
  // The operands of chunk c + 1 (W fragments, x chunk written and read back)
  // are read while chunk c's matrix steps run; the barrier that makes W
  // stage s + 1 visible comes at the start of stage s's last chunk, whose
  // fragments are already in registers.  Chunks 0 .. R-2 are in flight
  // before the loop.
#pragma unroll
  for (int i = 0; i < R - 1; ++i) load_chunk(i, xg[i]);
  sync();
  bf16x8 bc[CH], ac[CH];
  static_for<CH>([&](auto kc) { bc[decltype(kc)::value] = read_b(smem, decltype(kc)::value); });
  write_chunk(xg[0], 0);
  read_a(0);
#pragma unroll
  for (int kk = 0; kk < CH; ++kk) ac[kk] = af[kk];
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // U W stages; st0 is a multiple of U, so chunk c = st * CPS + cs has
  // c % R == (su * CPS + cs) % R and c % 2 == cs % 2.  Reads for a chunk
  // past the last are left unguarded in whole bodies (in-bounds LDS, never
  // consumed).
  const auto body = [&](int st0, auto guarded) {
    constexpr bool G = decltype(guarded)::value;
    static_for<U>([&](auto uc) {
      constexpr int su = decltype(uc)::value;
      const int st = st0 + su;
      if (!G || st < nst) {
        static_for<CPS>([&](auto ccs) {
          constexpr int cs = decltype(ccs)::value;
          constexpr int cl = su * CPS + cs;  // chunk within the body
          const int c = st * CPS + cs;
          if (!G || c < nch) {
            constexpr bool last = cs == CPS - 1;  // chunk c + 1 is in the next stage
            if (last && st + 1 < nst) sync();
            bf16x8 bn[CH];
            if (!G || c + 1 < nch) {
              const char *Bn = smem + ((last ? st + 1 : st) % S) * C::STAGE;
              static_for<CH>([&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                bn[kk] = read_b(Bn, ((cs + 1) % CPS) * CH + kk);
              });
              write_chunk(xg[(cl + 1) % R], (cs + 1) % 2);
              read_a((cs + 1) % 2);
            }
            // chunk c + R - 1 into the registers chunk c - 1 freed
            if (!G || c + R - 1 < nch) load_chunk(c + R - 1, xg[(cl + R - 1) % R]);
            static_for<CH>([&](auto kc) {
              constexpr int kk = decltype(kc)::value;
              if (!G || c * CH + kk < nk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ac[kk], bc[kk], acc, 0, 0, 0);
            });
#pragma unroll
            for (int kk = 0; kk < CH; ++kk) {
              bc[kk] = bn[kk];
              ac[kk] = af[kk];
            }
          }
        });
      }
    });
  };
  const int nfull = nk / (U * KS);
  for (int b = 0; b < nfull; ++b) body(b * U, std::false_type{});
  if (nfull * U * KS < nk) body(nfull * U, std::true_type{});
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = wave * 16 + g4 * 4 + q;
    if (m >= M) continue;
    if constexpr (sizeof(OutT) == 2) out[static_cast<int64_t>(m) * N + n0 + r16] = gemm_f32_to_bf16(acc[q]);
    else out[static_cast<int64_t>(m) * N + n0 + r16] = acc[q];
  }
}

// Buffer descriptors address 32-bit byte ranges: operands under 4 GiB take
// them, larger ones the 64-bit addresses.
static bool gemm_buf_ok(int64_t rows, int64_t K, int64_t N) {
  return rows * K * 2 < kBufFarOff && K * N * 2 < kBufFarOff;
}

// Rectangles per column of the XCD map (gemm_bf16_kernel): the gy in {1, 2,
// 4, 8} that divides the tile grid into eight equal rectangles with the fewest
// operand bytes per rectangle (rows x BM + columns x BN, both times K), or 0
// (the column-eighths map) when no such cut exists or the grid has fewer than
// two tiles per XCD.
static int gemm_xcd_rows(int64_t nx, int64_t ny, int bm, int bn) {
  if (nx * ny < 16) return 0;
  int best = 0;
  int64_t best_cost = 0;
  for (int gy = 1; gy <= 8; gy *= 2) {
    const int gx = 8 / gy;
    if (ny % gy != 0 || nx % gx != 0) continue;
    const int64_t cost = (ny / gy) * bm + (nx / gx) * bn;
    if (best == 0 || cost < best_cost) {
      best = gy;
      best_cost = cost;
    }
  }
  return best;
}

template <class C, class OutT = float>
static hipError_t launch_gemm_c(const uint16_t *x, const uint16_t *W, OutT *out, int64_t M, int64_t K,
                                int64_t N, hipStream_t stream) {
  const int64_t nx = N / C::BN, ny = (M + C::BM - 1) / C::BM;
  const dim3 grid(static_cast<uint32_t>(nx), static_cast<uint32_t>(ny));
  const int gy = gemm_xcd_rows(nx, ny, C::BM, C::BN);
  if (gemm_buf_ok(M, K, N))
    hipLaunchKernelGGL((gemm_bf16_kernel<C, OutT, true>), grid, dim3(C::NT), 0, stream, x, W, out, M,
                       static_cast<int>(K), static_cast<int>(N), gy);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<C, OutT, false>), grid, dim3(C::NT), 0, stream, x, W, out, M,
                       static_cast<int>(K), static_cast<int>(N), gy);
  return hipGetLastError();
}

template <int NC, class OutT>
static hipError_t launch_strip_nc(const uint16_t *x, const uint16_t *W, OutT *out, int64_t M, int64_t K, int64_t N,
                                  hipStream_t stream) {
  constexpr int S = NC <= 4 ? 8 : (160 * 1024 - NC * 8192) / 16384;
  using C = StripCfg<NC, 2, S, NC + 2 <= 8 ? 8 : 4>;
  hipLaunchKernelGGL((gemm_strip_kernel<C, OutT>), dim3(static_cast<uint32_t>(N / 16)), dim3(C::NT), 0, stream, x,
                     W, out, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N));
  return hipGetLastError();
}

// Batches of 1 .. 128 rows: one compute wavefront per 16-row fragment.
constexpr int64_t kStripMaxM = 128;
static bool strip_ok(int64_t M, int64_t K, int64_t N) {
  return M >= 1 && M <= kStripMaxM && M * K * 2 < 0x7FFFFFF0LL && gemm_buf_ok(M, K, N);
}

template <class OutT>
static hipError_t launch_strip(const uint16_t *x, const uint16_t *W, OutT *out, int64_t M, int64_t K, int64_t N,
                               hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return launch_strip_nc<1, OutT>(x, W, out, M, K, N, stream);
    case 2: return launch_strip_nc<2, OutT>(x, W, out, M, K, N, stream);
    case 3: return launch_strip_nc<3, OutT>(x, W, out, M, K, N, stream);
    case 4: return launch_strip_nc<4, OutT>(x, W, out, M, K, N, stream);
    case 5: return launch_strip_nc<5, OutT>(x, W, out, M, K, N, stream);
    case 6: return launch_strip_nc<6, OutT>(x, W, out, M, K, N, stream);
    case 7: return launch_strip_nc<7, OutT>(x, W, out, M, K, N, stream);
    default: return launch_strip_nc<8, OutT>(x, W, out, M, K, N, stream);
  }
}

// CT: a taller tile for experts of C::BM + 1 .. CT::BM rows, which then take
// one row tile instead of a full one and a ragged one (buffer-descriptor path
// only: with 64-bit addresses its registers spill)
template <class C, class CT = C>
static hipError_t launch_grouped_c(const uint16_t *x, int64_t Mx, const int32_t *rows, const uint16_t *W,
                                   const int32_t *offsets, int64_t E, int64_t P, int64_t K, int64_t N, float *out,
                                   hipStream_t stream) {
  // enough row tiles for any split of P rows over E experts, in eight
  // equal shares, each with all its column tiles (a tall tile takes the
  // place of two)
  const int64_t tiles = (P + C::BM - 1) / C::BM + E;
  const int64_t ncol = N / C::BN;
  const dim3 grid(static_cast<uint32_t>(8 * ((tiles + 7) / 8) * ncol));
  if (gemm_buf_ok(Mx, K, N))
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<C, CT, true>), grid, dim3(C::NT), 0, stream, x, Mx, rows, W,
                       offsets, static_cast<int>(E), P, out, static_cast<int>(K), static_cast<int>(N),
                       static_cast<int>(ncol));
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<C, C, false>), grid, dim3(C::NT), 0, stream, x, Mx, rows, W,
                       offsets, static_cast<int>(E), P, out, static_cast<int>(K), static_cast<int>(N),
                       static_cast<int>(ncol));
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_bf16(const uint16_t *x, int64_t Mx, const int32_t *rows, const uint16_t *W,
                                    const int32_t *offsets, int64_t E, int64_t P, int64_t K, int64_t N,
                                    float *out, hipStream_t stream) {
  // From 128 rows per expert on average, the dense kernel's large tile: at
  // 65536 rows x 2048 x 1024 over 256 experts of 193-324 rows it beats 128 x
  // 128 tiles (eight 32 x 64 wavefront tiles) by ~12% (configurations with
  // more stages in flight need more than the 256 registers a wavefront has
  // here).  Below that the weights dominate and 128 x 128 tiles stream them
  // faster: 22 vs 36 us at 8 rows, 169 vs 200 us at 512 rows (864 MiB of
  // weights, 5.3 TB/s), 220 vs 236 us at 16384 rows; at 32768 the large tile
  // wins (271 vs 289 us).  The large tile runs the rotated loop over
  // two-step stages: 416 against 430 us for the plain loop at 65536 rows.
  if (N % 256 == 0 && P >= 128 * E)
    return launch_grouped_c<GemmCfg<256, 256, 2, 4, 64, 2, true>, GemmCfg<320, 256, 2, 4, 64, 2, true>>(
        x, Mx, rows, W, offsets, E, P, K, N, out, stream);
  return launch_grouped_c<GemmCfg<128, 128, 4, 2, 64, 2>>(x, Mx, rows, W, offsets, E, P, K, N, out, stream);
}

// The tile is chosen from the shape (a performance choice only: every
// configuration runs the same per-output instruction sequence): the smallest
// tile whose count still fits the CUs, since a launch whose tiles all run at
// once takes about one tile's time.  In order: 32 x 32 (4 wavefronts, K in
// stages of 128 x 4) while there are at most two tiles per CU; 64 x 64 (4
// wavefronts, 128 x 3), 64 x 128 (8 wavefronts of 16 x 64, 64 x 2), 128 x
// 128 (8 of 32 x 64, 128 x 2) and 256 x 128 (8 of 64 x 64, 64 x 3) while
// their tiles fit the CUs once; else 256 x 256 (8 of 128 x 64, 64 x 2, the
// rotated loop: 121.6 against 130.4 us at M = K = N = 4096 with one-step
// stages in a ring of four, 219 against 241 at M = 8192).
// Measured against the best of the six at 30 shapes (M = 192..6144 at K = N
// = 4096, N = 256..14336): within ~1 us or 2% everywhere; e.g. K = N = 4096:
// M = 256 38 us, 512 43, 1024 56, 2048 90, 3072 124, 4096 142; K = 2048, N =
// 256: M = 1024 13 us, 8192 25.
// Small batches take the strip kernel (one 16-column strip of W with all
// the rows per workgroup) while its strips cover at least half the CUs and
// it measured faster: K = N = 4096, kernel time under a trace, M = 1 11.3
// us and M = 16 13.3 against 13.3 and 14.2 for 16-row strips of the dense
// stage layout; M = 112 and 128 20.7-21.3 against 22.2-22.6 for 32 x 32
// tiles.  From 17 to 96 rows the 32 x 32 tiles win (14.4-17.2 against
// 14.1-21.2 us): every strip reads all of x from L2, and at those sizes that
// broadcast, not W, sets the time.
template <class OutT>
static hipError_t launch_gemm_any(const uint16_t *x, const uint16_t *W, OutT *out, int64_t M, int64_t K, int64_t N,
                                  hipStream_t stream) {
  const int64_t cus = device_cus();
  const auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * (N / bn); };
  if ((M <= 16 || M > 96) && N / 16 >= cus / 2 && strip_ok(M, K, N))
    return launch_strip<OutT>(x, W, out, M, K, N, stream);
  if (M <= 128 || tiles(32, 32) <= 2 * cus)
    return launch_gemm_c<GemmCfg<32, 32, 2, 2, 128, 4>, OutT>(x, W, out, M, K, N, stream);
  if (tiles(64, 64) <= cus) return launch_gemm_c<GemmCfg<64, 64, 2, 2, 128, 3>, OutT>(x, W, out, M, K, N, stream);
  // two 32 KiB stages (64 KiB), so two workgroups share a CU and twice the tiles run
  // in one round; worth it while W, not x, is most of the traffic (M <= N):
  // 30.7 against 37.5 us at M = 512, K = N = 4096, but 30.0 against 23.7 at
  // M = 8192, K = 2048, N = 256, where each x row is read by more tiles
  if (tiles(64, 64) <= 2 * cus && M <= N)
    return launch_gemm_c<GemmCfg<64, 64, 2, 2, 128, 2>, OutT>(x, W, out, M, K, N, stream);
  if (tiles(64, 128) <= cus) return launch_gemm_c<GemmCfg<64, 128, 4, 2, 64, 2>, OutT>(x, W, out, M, K, N, stream);
  if (tiles(128, 128) <= cus) return launch_gemm_c<GemmCfg<128, 128, 4, 2, 128, 2>, OutT>(x, W, out, M, K, N, stream);
  if (tiles(256, 128) <= cus || N % 256 != 0)
    return launch_gemm_c<GemmCfg<256, 128, 4, 2, 64, 3>, OutT>(x, W, out, M, K, N, stream);
  return launch_gemm_c<GemmCfg<256, 256, 2, 4, 64, 2, true>, OutT>(x, W, out, M, K, N, stream);
}

hipError_t launch_gemm_bf16(const uint16_t *x, const uint16_t *W, float *out, int64_t M, int64_t K, int64_t N,
                            hipStream_t stream) {
  return launch_gemm_any<float>(x, W, out, M, K, N, stream);
}

// The same product with every output rounded to bf16 (round to nearest even):
// the logits of a router that runs its gate as a plain bf16 linear layer.
hipError_t launch_gemm_bf16_out_bf16(const uint16_t *x, const uint16_t *W, uint16_t *out, int64_t M, int64_t K,
                                     int64_t N, hipStream_t stream) {
  return launch_gemm_any<uint16_t>(x, W, out, M, K, N, stream);
}

}  // namespace drk
