// route_rowwise.hip -- the small-batch routing kernel.
//
// One workgroup of 256 threads routes T tokens.  Thread t owns experts
// t, t+256, ... and, for each of its outputs, runs the canonical order
// directly: a sequential fmaf chain from +0 over each 256-wide K-block (the
// block's x values staged in LDS and read as broadcasts, W rows read
// coalesced from global memory), each finished partial folded into the
// counter tree.  The E logits of a token then go through LDS to one
// wavefront, which ranks them and writes ids, weights and the margin.
//
// This is the "fixed reduction order per row, independent of how many rows
// share the launch" of "Batch changed the model's mind" (section "The fix:
// m-invariant twins"), on vector FMA; the tiled kernel computes the same
// operations on matrix cores.
#include "route_common.h"
#include "launch.h"

namespace drk {

constexpr int RW_THREADS = 256;
constexpr int RW_MAXL = 7;  // nb <= 64 (K <= 16384)

template <int E, int T>
__global__ __launch_bounds__(RW_THREADS) void route_rowwise_kernel(
    const float *__restrict__ xf, const uint16_t *__restrict__ xb, const float *__restrict__ W,
    int64_t M, int K, EpilogueArgs ea) {
  constexpr int NE = (E >= RW_THREADS) ? E / RW_THREADS : 1;
  __shared__ float xs[T][256];
  __shared__ float lg[T][E];

  const int t = threadIdx.x;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * T;
  const int nb = (K + 255) / 256;
  const bool active = (E >= RW_THREADS) || (t < E);

  float stk[RW_MAXL][T * NE];
  for (int b = 0; b < nb; ++b) {
    const int k0 = b * 256;
    const int len = (K - k0 < 256) ? (K - k0) : 256;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int64_t mm = m0 + i;
      float v = 0.0f;
      if (mm < M && t < len) {
        const int64_t off = mm * K + k0 + t;
        v = xb ? bf16_to_f32(xb[off]) : xf[off];
      }
      xs[i][t] = v;
    }
    __syncthreads();
    float p[T * NE];
#pragma unroll
    for (int o = 0; o < T * NE; ++o) p[o] = 0.0f;
    if (active) {
      const float *wrow = W + static_cast<int64_t>(k0) * E + t;
#pragma unroll 4
      for (int kk = 0; kk < len; ++kk) {
#pragma unroll
        for (int q = 0; q < NE; ++q) {
          const float w = wrow[static_cast<int64_t>(kk) * E + q * RW_THREADS];
#pragma unroll
          for (int i = 0; i < T; ++i) p[i * NE + q] = __builtin_fmaf(xs[i][kk], w, p[i * NE + q]);
        }
      }
    }
    tree_push<RW_MAXL, T * NE>(stk, p, b);
  }
  float out[T * NE];
  tree_final<RW_MAXL, T * NE>(stk, nb, out);
  if (active) {
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
      for (int q = 0; q < NE; ++q) lg[i][t + q * RW_THREADS] = out[i * NE + q];
  }
  __syncthreads();
  const int wave = t >> 6;
  for (int i = wave; i < T; i += RW_THREADS / 64) {
    const int64_t mm = m0 + i;
    if (mm < M) route_token<E>(lg[i], mm, ea);
  }
}

template <int E, int T>
static hipError_t launch_rowwise_t(const RouteLaunch &L) {
  const int64_t nblk = (L.M + T - 1) / T;
  EpilogueArgs ea{L.k, L.logit_bf16, L.flags, L.ids, L.weights, L.logits, L.margins};
  hipLaunchKernelGGL((route_rowwise_kernel<E, T>), dim3(static_cast<uint32_t>(nblk)), dim3(RW_THREADS), 0,
                     L.stream, L.xf, L.xb, L.W, L.M, static_cast<int>(L.K), ea);
  return hipGetLastError();
}

template <int E>
static hipError_t launch_rowwise_e(const RouteLaunch &L) {
  // tokens per workgroup from M only: one token per wavefront at small M so
  // more workgroups share the W stream, more per workgroup as M grows
  if constexpr (E >= 512) {
    return launch_rowwise_t<E, 4>(L);
  } else {
    if (L.M <= 256) return launch_rowwise_t<E, 4>(L);
    return launch_rowwise_t<E, 8>(L);
  }
}

hipError_t launch_route_rowwise(const RouteLaunch &L) {
  switch (L.E) {
    case 64: return launch_rowwise_e<64>(L);
    case 128: return launch_rowwise_e<128>(L);
    case 256: return launch_rowwise_e<256>(L);
    case 512: return launch_rowwise_e<512>(L);
    case 1024: return launch_rowwise_e<1024>(L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace drk
