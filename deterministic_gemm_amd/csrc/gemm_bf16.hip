// gemm_bf16.hip -- batch-invariant dense GEMM on bf16 matrix cores.
//
// out[M,N] = x[M,K] . W[K,N], bf16 inputs, fp32 accumulation.  A batch-
// invariant kernel must reduce K in one static order whatever the shape ("The
// Illusion of Determinism in Disaggregated Inference", section "The arithmetic
// cost of batch-invariant kernels").  Every output here is accumulated by the
// same instruction sequence: one v_mfma_f32_16x16x32_bf16 per 32-wide K step,
// k ascending, into one accumulator that starts at zero, with no split of K.
// The tile over M and N only decides which lanes run that sequence, so a row
// gets the same bits at every M and at every position in a tile.  The
// matrix core's internal order of the 32 products of one step is the
// hardware's; results are therefore compared with the exact product within a
// tolerance, and with themselves across M bit for bit.
//
// Workgroup tile 128x128, four wavefronts of 64x64 (4x4 MFMA tiles), K staged
// through LDS 32 at a time: x as [row][k], W transposed to [n][k] so that each
// lane reads eight consecutive k of its column.
#include "launch.h"

namespace drk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int GB_M = 128, GB_N = 128, GB_K = 32, GB_T = 256;
constexpr int GB_P = GB_K + 8;  // LDS row pitch in bf16 elements

__global__ __launch_bounds__(GB_T) void gemm_bf16_kernel(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ W,
                                                         float *__restrict__ out, int64_t M, int K,
                                                         int N) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GB_M * GB_P];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[GB_N * GB_P];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * GB_M;
  const int n0 = blockIdx.x * GB_N;
  const int r16 = lane & 15, g4 = lane >> 4;

  uint4 areg[2], breg[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + GB_T * i;
      const int row = c >> 2, kc = (c & 3) * 8;
      const int64_t m = m0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < M) v = *reinterpret_cast<const uint4 *>(x + m * K + k0 + kc);
      areg[i] = v;
      const int kr = c >> 4, nc = (c & 15) * 8;
      breg[i] = *reinterpret_cast<const uint4 *>(W + static_cast<int64_t>(k0 + kr) * N + n0 + nc);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + GB_T * i;
      const int row = c >> 2, kc = (c & 3) * 8;
      *reinterpret_cast<uint4 *>(&As[row * GB_P + kc]) = areg[i];
      const int kr = c >> 4, nc = (c & 15) * 8;
      const uint32_t w4[4] = {breg[i].x, breg[i].y, breg[i].z, breg[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Bs[(nc + 2 * j) * GB_P + kr] = static_cast<uint16_t>(w4[j] & 0xFFFFu);
        Bs[(nc + 2 * j + 1) * GB_P + kr] = static_cast<uint16_t>(w4[j] >> 16);
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  load(0);
  for (int k0 = 0; k0 < K; k0 += GB_K) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + GB_K < K) load(k0 + GB_K);
    bf16x8 af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm * 64 + i * 16 + r16) * GB_P + g4 * 8]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn * 64 + j * 16 + r16) * GB_P + g4 * 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = m0 + wm * 64 + i * 16 + g4 * 4 + q;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[m * N + n0 + wn * 64 + j * 16 + r16] = acc[i][j][q];
    }
}

hipError_t launch_gemm_bf16(const uint16_t *x, const uint16_t *W, float *out, int64_t M,
                            int64_t K, int64_t N, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(N / GB_N), static_cast<uint32_t>((M + GB_M - 1) / GB_M));
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(GB_T), 0, stream, x, W, out, M, static_cast<int>(K),
                     static_cast<int>(N));
  return hipGetLastError();
}

}  // namespace drk
