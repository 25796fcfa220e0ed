// route_tiny.hip -- the logits for batches of a few tokens, on the vector ALUs.
//
// A matrix-core step of the canonical chain issues only after the previous
// one completes (about 40 clocks for a dependent fp32 MFMA on gfx950), so the
// 256 steps of one K-block cost several microseconds however few tokens there
// are.  A dependent vector fmaf issues every few clocks.  This family gives
// each lane one (expert, K-block) chain per token -- fmaf from +0 over the
// block's k ascending ("Batch changed the model's mind", section "The fix:
// m-invariant twins": a fixed reduction order per row) -- and combines the
// blocks of an expert across lanes by a xor butterfly, which is the pairwise
// tree over -0-padded block partials ("The Illusion of Determinism in
// Disaggregated Inference", section "The anatomy of the missing numeric
// contract").  The selection kernel then runs on the stored logits.
//
// A workgroup holds NW wavefronts, one token each, that share one W slice:
// P = the next power of two >= nb block slots, 64 / P experts.  The slice (K
// rows of 64/P experts, 64 KiB at most), its transfers dealt out to the NW
// wavefronts, and each wavefront's x row go to LDS in one burst of
// global_load_lds_dwordx4 transfers; each block's rows are followed by one
// row of padding, so the P blocks read at one k land on distinct LDS banks.
#include "route_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace drk {

template <int P, int NW>
struct TinyCfg {
  static_assert(P >= 1 && P <= 16 && (P & (P - 1)) == 0, "block slots");
  static_assert(NW >= 1 && NW <= 8, "wavefronts");
  static constexpr int EPW = 64 / P;                 // experts per workgroup
  static constexpr int ROWB = EPW * 4;               // bytes of one W row slice
  static constexpr int WBLK = 256 * ROWB + ROWB;     // one block of rows plus a padding row
  static constexpr int XBLK = 1024 + 16;             // 256 values of one token's block plus padding
  static constexpr int WBYTES = P * WBLK;
  static constexpr int XBYTES = NW * P * XBLK;       // one token per wavefront
  static constexpr int RPI = 1024 / ROWB;            // W rows per transfer instruction
  static_assert(WBYTES + XBYTES <= 160 * 1024, "LDS");
};

// the most wavefronts a workgroup's LDS leaves room for
template <int P>
constexpr int kTinyMaxNW = P <= 8 ? 8 : 4;

// XB: x holds bf16 bits (K % 8 == 0), staged as they are and widened
// exactly when read; else fp32 (K % 4 == 0).
template <int P, int NW, bool XB>
__global__ __launch_bounds__(64 * NW) void route_tiny_logits_kernel(const void *__restrict__ xv,
                                                                    const float *__restrict__ W, int64_t M, int K,
                                                                    int E, int logit_bf16, void *__restrict__ logits) {
  using C = TinyCfg<P, NW>;
  __shared__ __attribute__((aligned(16))) char smem[C::WBYTES + C::XBYTES];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char *wl = smem, *xl = smem + C::WBYTES + wave * (P * C::XBLK);
  const int ng = gridDim.x;
  const int g = (ng % 8 == 0) ? (blockIdx.x % 8) * (ng / 8) + blockIdx.x / 8 : blockIdx.x;  // XCD-contiguous groups
  const int e0 = g * C::EPW;
  const int64_t m = static_cast<int64_t>(blockIdx.y) * NW + wave;  // this wavefront's token
  const int nb = (K + 255) / 256;

  // W slice: block b's rows k = 256 b .. 256 b + 255, ROWB bytes each, its
  // transfer instructions dealt out to the NW wavefronts in turn.  At most
  // 32 transfers stay outstanding (the wait counter holds 63).
  int issued = 0;
  for (int b = 0; b < nb; ++b)
    for (int i = 0; i < 256 / C::RPI; ++i) {
      if ((b * (256 / C::RPI) + i) % NW != wave) continue;
      if (++issued > 32) wait_vmcnt<31>();
      const int r = i * C::RPI + lane / (C::ROWB / 16);  // row within the block
      const int u = lane % (C::ROWB / 16);               // 16-byte unit within the row
      const int kk = 256 * b + r;
      const void *src = &g_pad_pos;
      if (kk < K) src = W + static_cast<int64_t>(kk) * E + e0 + 4 * u;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<const float *>(wl + b * C::WBLK + i * 1024))));
    }
  // the token's x row: block b's 256 values in one instruction (bf16: the
  // first 32 lanes; the others fill the block's unused upper half)
  for (int b = 0; b < nb; ++b) {
    if (++issued > 32) wait_vmcnt<31>();
    const int kk = 256 * b + (XB ? 8 : 4) * lane;
    const void *src = &g_pad_pos;
    if (m < M && kk < K && (!XB || lane < 32)) {
      if constexpr (XB) src = static_cast<const uint16_t *>(xv) + m * K + kk;
      else src = static_cast<const float *>(xv) + m * K + kk;
    }
    dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<const float *>(xl + b * C::XBLK))));
  }
  compiler_fence();
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();  // the W slice came from every wavefront
  compiler_fence();

  const int b = lane / C::EPW, e = lane % C::EPW;
  const int klen = (b < nb) ? min(256, K - 256 * b) : 0;  // a multiple of 4
  float acc = (b < nb) ? 0.0f : -0.0f;
  const float *wrow = reinterpret_cast<const float *>(wl + b * C::WBLK) + e;
  const char *xrow = xl + b * C::XBLK;
  // unrolled so that later steps' LDS reads are in flight while a step's
  // fmafs wait on their operands
#pragma unroll 8
  for (int k = 0; k < klen; k += 4) {
    float4 xk;
    if constexpr (XB) {
      const uint2 u = *reinterpret_cast<const uint2 *>(xrow + 2 * k);  // four bf16, little-endian pairs
      xk = make_float4(u2f(u.x << 16), u2f(u.x & 0xFFFF0000u), u2f(u.y << 16), u2f(u.y & 0xFFFF0000u));
    } else {
      xk = *reinterpret_cast<const float4 *>(xrow + 4 * k);
    }
    acc = __builtin_fmaf(xk.x, wrow[(k + 0) * C::EPW], acc);
    acc = __builtin_fmaf(xk.y, wrow[(k + 1) * C::EPW], acc);
    acc = __builtin_fmaf(xk.z, wrow[(k + 2) * C::EPW], acc);
    acc = __builtin_fmaf(xk.w, wrow[(k + 3) * C::EPW], acc);
  }
  // the tree over the P block slots: level d adds lanes whose block index
  // differs in bit d, adjacent blocks first
#pragma unroll
  for (int d = C::EPW; d < 64; d <<= 1) acc = acc + __shfl_xor(acc, d, 64);
  if (b == 0 && m < M) {
    if (logit_bf16) static_cast<uint16_t *>(logits)[m * E + e0 + e] = f32_to_bf16(acc);
    else static_cast<float *>(logits)[m * E + e0 + e] = acc;
  }
}

template <int P, int NW>
static hipError_t launch_tiny_pw(const RouteLaunch &L) {
  const dim3 grid(static_cast<uint32_t>(L.E / TinyCfg<P, NW>::EPW), static_cast<uint32_t>((L.M + NW - 1) / NW));
  if (L.xf)
    hipLaunchKernelGGL((route_tiny_logits_kernel<P, NW, false>), grid, dim3(64 * NW), 0, L.stream,
                       static_cast<const void *>(L.xf), L.W, L.M, static_cast<int>(L.K), static_cast<int>(L.E),
                       L.logit_bf16, L.logits);
  else
    hipLaunchKernelGGL((route_tiny_logits_kernel<P, NW, true>), grid, dim3(64 * NW), 0, L.stream,
                       static_cast<const void *>(L.xb), L.W, L.M, static_cast<int>(L.K), static_cast<int>(L.E),
                       L.logit_bf16, L.logits);
  return hipGetLastError();
}

// The LDS of one workgroup admits one per CU.  Four wavefronts while the
// workgroups fit the CUs at once, else as many as LDS allows.  Measured at
// K=2048, E=256, logits kernel alone: 6.0-6.4 us for M=1..32 with four
// wavefronts (one wavefront per workgroup with four tokens each: 7.2-11.4),
// 7.2-7.9 us for M=33..64 with eight; at K=4096: 6.4-8.3 us for M=1..16.
template <int P>
static hipError_t launch_tiny_p(const RouteLaunch &L) {
  const int64_t groups = L.E / TinyCfg<P, 4>::EPW;
  if constexpr (kTinyMaxNW<P> > 4) {
    if (groups * ((L.M + 3) / 4) > device_cus()) return launch_tiny_pw<P, kTinyMaxNW<P>>(L);
  }
  return launch_tiny_pw<P, 4>(L);
}

bool tiny_supports(int64_t E, int64_t K, bool x_f32, bool has_logits) {
  return has_logits && K % (x_f32 ? 4 : 8) == 0 && K <= 4096 && E % 64 == 0 && E <= 1024;
}

hipError_t launch_route_tiny_logits(const RouteLaunch &L) {
  const int64_t nb = (L.K + 255) / 256;
  // A batch of a few tokens streams all of W through E * P / 64 workgroups.
  // Sixteen block slots (four experts per workgroup; slots past nb hold -0,
  // which leaves every sum as it is) spread it over more of them, each with
  // a smaller slice, while they fill at most half the CUs.  Measured at K =
  // 2048, E = 256, whole route: 9.9 against 10.5 us at M = 1, 10.6 against
  // 11.2 at M = 4, 10.7 against 11.2 at M = 8; at M = 16, where they would
  // fill every CU, 11.8 against 11.5.
  if (nb <= 16 && (L.E / 4) * ((L.M + 3) / 4) <= device_cus() / 2) return launch_tiny_p<16>(L);
  if (nb <= 1) return launch_tiny_p<1>(L);
  if (nb <= 2) return launch_tiny_p<2>(L);
  if (nb <= 4) return launch_tiny_p<4>(L);
  if (nb <= 8) return launch_tiny_p<8>(L);
  return launch_tiny_p<16>(L);
}

hipError_t launch_route_tiny(const RouteLaunch &L) {
  const hipError_t e = launch_route_tiny_logits(L);
  if (e != hipSuccess) return e;
  return launch_route_select(L);
}

// Batches this family takes: while its workgroups, with as many wavefronts as
// LDS allows, fit the CUs at once; past that a second round of workgroups
// costs as much as the first, and the narrow family is faster.  Where the
// narrow family does not take E but the two-kernel family does (E = 1024),
// up to 64 tokens at K <= 2048 and 32 above: measured at E = 1024 (full
// route), 42 against 59 us at M = 64 and 68 against 59 at M = 128 (K =
// 2048); 73 against 101 at M = 32 and 125 against 99 at M = 64 (K = 4096).
// Where neither does, up to 4096 tokens against the row-wise family, the one
// left (E = 1024, K = 2048: 128 against 1917 us at M = 256).
int64_t tiny_max_m(int64_t E, int64_t K) {
  if (!narrow_supports(E, K, true, true)) return split_supports(E, K, true, true) ? (K <= 2048 ? 64 : 32) : 4096;
  int p = 1;
  while (p < (K + 255) / 256) p <<= 1;
  const int64_t nw = p <= 8 ? 8 : 4, groups = E * p / 64;
  return groups > 0 ? nw * (device_cus() / groups) : 0;
}

}  // namespace drk
