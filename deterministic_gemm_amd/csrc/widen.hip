// widen.hip -- bf16 activations widened exactly to fp32.
//
// A bf16 value is the upper half of the fp32 bit pattern of the same number,
// so the widening is a 16-bit shift with no rounding, and routing the widened
// rows gives the bits that routing the bf16 rows does (x "widened exactly" is
// the router's input contract for bf16 activations).  The fp32 router families
// stage x through LDS in 16-byte units of four values; this pass lets bf16
// callers reach them.  Bound by HBM: 6 bytes per element (2 read, 4 written).
#include "launch.h"

namespace drk {

__global__ __launch_bounds__(256) void widen_bf16_kernel(const uint16_t *__restrict__ x, int64_t n,
                                                         float *__restrict__ out) {
  const int64_t n8 = n / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 u = reinterpret_cast<const uint4 *>(x)[i];  // eight bf16, little-endian pairs
    reinterpret_cast<uint4 *>(out)[2 * i] = make_uint4(u.x << 16, u.x & 0xFFFF0000u, u.y << 16, u.y & 0xFFFF0000u);
    reinterpret_cast<uint4 *>(out)[2 * i + 1] =
        make_uint4(u.z << 16, u.z & 0xFFFF0000u, u.w << 16, u.w & 0xFFFF0000u);
  }
  // the last n % 8 elements
  if (blockIdx.x == 0 && threadIdx.x < n - 8 * n8) {
    const int64_t t = 8 * n8 + threadIdx.x;
    out[t] = __uint_as_float(static_cast<uint32_t>(x[t]) << 16);
  }
}

hipError_t launch_widen_bf16(const uint16_t *x, int64_t n, float *out, hipStream_t stream) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, x, n, out);
  return hipGetLastError();
}

}  // namespace drk
