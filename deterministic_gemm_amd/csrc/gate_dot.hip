// gate_dot.hip -- the shared-expert gate: a one-output canonical dot per row
// followed by a sigmoid.  "Batch changed the model's mind" (section "m-scan:
// the staircase") found this one-output dot drifting between m=74 and m=75
// under a shape-dependent library GEMM; here it is the router's canonical
// order with E = 1, so it cannot move with M.
//
// One wavefront per row: lane b runs the fmaf chain of K-block b (nb <= 64
// lanes), lanes past the last block hold -0.0, and the 64 partials are
// combined by a xor butterfly -- level d adds lanes that differ in bit d, which
// is the pairwise tree over the -0-padded leaves.
#include "route_common.h"
#include "launch.h"

namespace drk {

constexpr int GD_WAVES = 4;

template <bool XB, bool WB>
__global__ __launch_bounds__(GD_WAVES * 64) void gate_dot_kernel(const void *__restrict__ x,
                                                                  const void *__restrict__ w,
                                                                  float *__restrict__ dot,
                                                                  float *__restrict__ gate, int64_t M,
                                                                  int K) {
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * GD_WAVES + (threadIdx.x >> 6);
  if (m >= M) return;
  const int nb = (K + 255) / 256;
  float p = -0.0f;
  if (lane < nb) {
    p = 0.0f;
    const int k0 = lane * 256;
    const int k1 = (K - k0 < 256) ? K : k0 + 256;
    for (int kk = k0; kk < k1; ++kk) {
      const int64_t off = m * K + kk;
      const float xv = XB ? bf16_to_f32(static_cast<const uint16_t *>(x)[off]) : static_cast<const float *>(x)[off];
      const float wv = WB ? bf16_to_f32(static_cast<const uint16_t *>(w)[kk]) : static_cast<const float *>(w)[kk];
      p = __builtin_fmaf(xv, wv, p);
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) p = p + __shfl_xor(p, d, 64);
  if (lane == 0) {
    if (dot) dot[m] = p;
    if (gate) {
      const float e = route_exp(-__builtin_fabsf(p));
      gate[m] = (p >= 0.0f) ? 1.0f / (1.0f + e) : e / (1.0f + e);
    }
  }
}

hipError_t launch_gate_dot(const void *x, int x_bf16, const void *w, int w_bf16, float *dot,
                           float *gate, int64_t M, int64_t K, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((M + GD_WAVES - 1) / GD_WAVES)), block(GD_WAVES * 64);
  const int k = static_cast<int>(K);
  if (x_bf16 && w_bf16)
    hipLaunchKernelGGL((gate_dot_kernel<true, true>), grid, block, 0, stream, x, w, dot, gate, M, k);
  else if (x_bf16)
    hipLaunchKernelGGL((gate_dot_kernel<true, false>), grid, block, 0, stream, x, w, dot, gate, M, k);
  else if (w_bf16)
    hipLaunchKernelGGL((gate_dot_kernel<false, true>), grid, block, 0, stream, x, w, dot, gate, M, k);
  else
    hipLaunchKernelGGL((gate_dot_kernel<false, false>), grid, block, 0, stream, x, w, dot, gate, M, k);
  return hipGetLastError();
}

}  // namespace drk
