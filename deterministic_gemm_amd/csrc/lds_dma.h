// lds_dma.h -- global-to-LDS transfers for the pipelined routing kernels:
// the transfer instruction itself, the vector-memory wait, and the padding
// vectors that out-of-range lanes read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace drk {

// 16-byte padding read by lanes whose element lies past the end of x or W:
// x pads with +0.0 and W with -0.0, so the padded product is -0.0, the
// identity of addition, and fma(+0, -0, c) == c leaves every chain unchanged.
struct Pad16 {
  float v[4];
};
static __device__ const Pad16 g_pad_pos = {{0.0f, 0.0f, 0.0f, 0.0f}};
static __device__ const Pad16 g_pad_neg = {{-0.0f, -0.0f, -0.0f, -0.0f}};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt with only the LDS counter constrained, to zero (gfx9 encoding).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// One global -> LDS transfer: every active lane moves the 16 bytes at `src`
// to LDS address lds_base + 16 * lane.  Written as inline assembly so that
// the compiler's wait-count pass does not treat it as an LDS write to be
// drained before every LDS read; the kernel orders these transfers itself
// (wait_vmcnt + barrier).  The LDS base goes in as an m0 operand ("{m0}"), so
// the compiler writes m0 itself and knows the statement reads it: no value
// of its own is ever kept in m0 across the transfer.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_base) : "memory");
}

// The same transfer addressed as a 64-bit SGPR base plus a 32-bit per-lane
// byte offset: half the per-lane address operand, which measurably reduces the
// time each transfer takes from the matrix cores' issue.
__device__ __forceinline__ void dma16_s(const float *base, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_base) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const float *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

}  // namespace drk
