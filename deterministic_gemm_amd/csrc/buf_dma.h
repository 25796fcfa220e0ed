// buf_dma.h -- global-to-LDS transfers through buffer descriptors: a
// uniform 128-bit descriptor (base, byte range) plus one 32-bit byte offset
// per lane.  A lane whose offset lies past the range reads zeros without
// touching memory (checked per 4-byte word), which takes the place of
// padding reads; the offsets take half the registers of 64-bit addresses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace drk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kBufFarOff = 0xFFFFFFF0u;  // past every range

__device__ __forceinline__ u32x4 buf_rsrc(const void *base, int64_t nbytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t n = nbytes <= 0 ? 0 : (nbytes >= kBufFarOff ? kBufFarOff : static_cast<uint64_t>(nbytes));
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));  // stride 0: a raw byte range
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(n));
  r[3] = 0x00020000u;
  return r;
}

// Every active lane moves the 16 bytes at byte offset voff of the descriptor's
// range (zeros past it) to LDS address lds_base + 16 * lane; inline assembly
// for the reason given at dma16, with the LDS base as an m0 operand likewise.
__device__ __forceinline__ void dma16_buf(uint32_t voff, u32x4 rsrc, uint32_t lds_base) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base) : "memory");
}

}  // namespace drk
