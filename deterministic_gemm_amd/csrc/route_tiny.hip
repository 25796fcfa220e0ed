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
// One wavefront per workgroup: P = the next power of two >= nb block slots,
// 64 / P experts, T tokens.  The workgroup's whole W slice (K rows of 64/P
// experts, 64 KiB at most) and its tokens' x rows go to LDS in one burst of
// global_load_lds_dwordx4 transfers; each block's rows are followed by one
// row of padding, so the P blocks read at one k land on distinct LDS banks.
#include "route_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace drk {

// Batches this family takes: up to 48 tokens when a workgroup's W slice
// leaves room for six tokens' x (K <= 2048) and E <= 512, else 32.  Measured at K=2048,
// E=256, logits kernel alone: 10.1 us at M=32 (four tokens per workgroup),
// 12.2 us at M=40..48 with six (four: 19.0; the narrow family: 14.7), 14.9 us
// at M=64 with eight (narrow: 14.8).
constexpr int64_t kTinyMaxM = 32, kTinyMaxM6 = 48;

template <int P, int T>
struct TinyCfg {
  static_assert(P >= 1 && P <= 16 && (P & (P - 1)) == 0, "block slots");
  static constexpr int EPW = 64 / P;                 // experts per workgroup
  static constexpr int ROWB = EPW * 4;               // bytes of one W row slice
  static constexpr int WBLK = 256 * ROWB + ROWB;     // one block of rows plus a padding row
  static constexpr int XBLK = 1024 + 16;             // 256 values of one token's block plus padding
  static constexpr int WBYTES = P * WBLK;
  static constexpr int XBYTES = T * P * XBLK;
  static constexpr int RPI = 1024 / ROWB;            // W rows per transfer instruction
  static_assert(WBYTES + XBYTES <= 160 * 1024, "LDS");
};

template <int P, int T>
__global__ __launch_bounds__(64) void route_tiny_logits_kernel(const float *__restrict__ x,
                                                               const float *__restrict__ W, int64_t M, int K,
                                                               int E, int logit_bf16, void *__restrict__ logits) {
  using C = TinyCfg<P, T>;
  __shared__ __attribute__((aligned(16))) char smem[C::WBYTES + C::XBYTES];
  char *wl = smem, *xl = smem + C::WBYTES;
  const int lane = threadIdx.x;
  const int ng = gridDim.x;
  const int g = (ng % 8 == 0) ? (blockIdx.x % 8) * (ng / 8) + blockIdx.x / 8 : blockIdx.x;  // XCD-contiguous groups
  const int e0 = g * C::EPW;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * T;
  const int nb = (K + 255) / 256;

  // W slice: block b's rows k = 256 b .. 256 b + 255, ROWB bytes each.  At
  // most 32 transfers stay outstanding (the wait counter holds 63).
  int issued = 0;
  for (int b = 0; b < nb; ++b)
    for (int i = 0; i < 256 / C::RPI; ++i) {
      if (++issued > 32) wait_vmcnt<31>();
      const int r = i * C::RPI + lane / (C::ROWB / 16);  // row within the block
      const int u = lane % (C::ROWB / 16);               // 16-byte unit within the row
      const int kk = 256 * b + r;
      const void *src = &g_pad_pos;
      if (kk < K) src = W + static_cast<int64_t>(kk) * E + e0 + 4 * u;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<const float *>(wl + b * C::WBLK + i * 1024))));
    }
  // x rows: token t, block b: 256 values in one instruction
  for (int t = 0; t < T; ++t)
    for (int b = 0; b < nb; ++b) {
      if (++issued > 32) wait_vmcnt<31>();
      const int kk = 256 * b + 4 * lane;
      const void *src = &g_pad_pos;
      if (m0 + t < M && kk < K) src = x + (m0 + t) * K + kk;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<const float *>(xl + (t * P + b) * C::XBLK))));
    }
  compiler_fence();
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();

  const int b = lane / C::EPW, e = lane % C::EPW;
  const int klen = (b < nb) ? min(256, K - 256 * b) : 0;  // a multiple of 4
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = (b < nb) ? 0.0f : -0.0f;
  const float *wrow = reinterpret_cast<const float *>(wl + b * C::WBLK) + e;
  const float *xrow = reinterpret_cast<const float *>(xl + b * C::XBLK);
  // unrolled so that later steps' LDS reads are in flight while a step's
  // fmafs wait on their operands
#pragma unroll 8
  for (int k = 0; k < klen; k += 4) {
    const float w0 = wrow[(k + 0) * C::EPW], w1 = wrow[(k + 1) * C::EPW];
    const float w2 = wrow[(k + 2) * C::EPW], w3 = wrow[(k + 3) * C::EPW];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float4 xv = *reinterpret_cast<const float4 *>(xrow + t * (P * C::XBLK / 4) + k);
      acc[t] = __builtin_fmaf(xv.x, w0, acc[t]);
      acc[t] = __builtin_fmaf(xv.y, w1, acc[t]);
      acc[t] = __builtin_fmaf(xv.z, w2, acc[t]);
      acc[t] = __builtin_fmaf(xv.w, w3, acc[t]);
    }
  }
  // the tree over the P block slots: level d adds lanes whose block index
  // differs in bit d, adjacent blocks first
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float v = acc[t];
#pragma unroll
    for (int d = C::EPW; d < 64; d <<= 1) v = v + __shfl_xor(v, d, 64);
    acc[t] = v;
  }
  if (b == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t m = m0 + t;
      if (m >= M) break;
      if (logit_bf16) static_cast<uint16_t *>(logits)[m * E + e0 + e] = f32_to_bf16(acc[t]);
      else static_cast<float *>(logits)[m * E + e0 + e] = acc[t];
    }
  }
}

template <int P, int T>
static hipError_t launch_tiny_pt(const RouteLaunch &L) {
  const dim3 grid(static_cast<uint32_t>(L.E / TinyCfg<P, T>::EPW), static_cast<uint32_t>((L.M + T - 1) / T));
  hipLaunchKernelGGL((route_tiny_logits_kernel<P, T>), grid, dim3(64), 0, L.stream, L.xf, L.W, L.M,
                     static_cast<int>(L.K), static_cast<int>(L.E), L.logit_bf16, L.logits);
  return hipGetLastError();
}

template <int P>
static hipError_t launch_tiny_p(const RouteLaunch &L) {
  if (L.M <= 1) return launch_tiny_pt<P, 1>(L);
  if (L.M <= 2) return launch_tiny_pt<P, 2>(L);
  if constexpr (P <= 8) {
    if (L.M > kTinyMaxM) return launch_tiny_pt<P, 6>(L);
  }
  return launch_tiny_pt<P, 4>(L);
}

bool tiny_supports(int64_t E, int64_t K, bool x_f32, bool has_logits) {
  return x_f32 && has_logits && K % 4 == 0 && K <= 4096 && E % 64 == 0 && E <= 1024;
}

hipError_t launch_route_tiny_logits(const RouteLaunch &L) {
  const int64_t nb = (L.K + 255) / 256;
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

int64_t tiny_max_m(int64_t E, int64_t K) { return ((K + 255) / 256 <= 8 && E <= 512) ? kTinyMaxM6 : kTinyMaxM; }

}  // namespace drk
