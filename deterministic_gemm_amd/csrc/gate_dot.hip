// gate_dot.hip -- the shared-expert gate: a one-output canonical dot per row
// followed by a sigmoid.  "Batch changed the model's mind" (section "m-scan:
// the staircase") found this one-output dot drifting between m=74 and m=75
// under a shape-dependent library GEMM; here it is the router's canonical
// order with E = 1, so it cannot move with M.
//
// Lanes per row = the next power of two >= nb (<= 64), so a wavefront takes
// 64 / that many rows: lane b of a row group runs the fmaf chain of K-block b
// (lanes past the last block hold -0.0), and the group's partials combine by a
// xor butterfly over its lanes -- level d adds lanes that differ in bit d,
// which is the pairwise tree over the -0-padded leaves.  Each lane streams its
// block with 16-byte loads (eight bf16 or four fp32 values per load) when rows
// are 16-byte aligned, and element by element otherwise; the path is bound by
// HBM (M*K elements of x read once).
#include "route_common.h"
#include "lds_dma.h"
#include "launch.h"

namespace drk {

constexpr int GD_WAVES = 4;

template <bool B>
__device__ __forceinline__ float load_elem(const void *p, int64_t i) {
  if constexpr (B) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

// Widen one 16-byte piece: 8 bf16 or 4 fp32 values.
template <bool B>
__device__ __forceinline__ void unpack16(const uint4 &u, float (&v)[B ? 8 : 4]) {
  if constexpr (B) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = u2f(w[j] << 16);
      v[2 * j + 1] = u2f(w[j] & 0xFFFF0000u);
    }
  } else {
    v[0] = u2f(u.x);
    v[1] = u2f(u.y);
    v[2] = u2f(u.z);
    v[3] = u2f(u.w);
  }
}

template <bool XB, bool WB, int LPR>
__global__ __launch_bounds__(GD_WAVES * 64) void gate_dot_kernel(const void *__restrict__ x,
                                                                  const void *__restrict__ w,
                                                                  float *__restrict__ dot,
                                                                  float *__restrict__ gate, int64_t M,
                                                                  int K, int vec) {
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int b = lane % LPR;
  const int64_t m = (static_cast<int64_t>(blockIdx.x) * GD_WAVES + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int nb = (K + 255) / 256;
  float p = -0.0f;
  if (m < M && b < nb) {
    p = 0.0f;
    const int k0 = b * 256;
    const int k1 = (K - k0 < 256) ? K : k0 + 256;
    int kk = k0;
    if constexpr (XB == WB) {
      // both operands in 16-byte pieces of the same element count
      constexpr int PE = XB ? 8 : 4;
      if (vec) {
        const uint4 *xs =
            reinterpret_cast<const uint4 *>(static_cast<const char *>(x) + (m * K + k0) * (XB ? 2 : 4));
        const uint4 *ws =
            reinterpret_cast<const uint4 *>(static_cast<const char *>(w) + static_cast<int64_t>(k0) * (WB ? 2 : 4));
        const int np = (k1 - k0) / PE;
#pragma unroll 4
        for (int i = 0; i < np; ++i) {
          float xv[PE], wv[PE];
          unpack16<XB>(xs[i], xv);
          unpack16<WB>(ws[i], wv);
#pragma unroll
          for (int j = 0; j < PE; ++j) p = __builtin_fmaf(xv[j], wv[j], p);
        }
        kk = k0 + np * PE;
      }
    }
    for (; kk < k1; ++kk) p = __builtin_fmaf(load_elem<XB>(x, m * K + kk), load_elem<WB>(w, kk), p);
  }
#pragma unroll
  for (int d = 1; d < LPR; d <<= 1) p = p + __shfl_xor(p, d, 64);
  if (m < M && b == 0) {
    if (dot) dot[m] = p;
    if (gate) {
      const float e = route_exp(-__builtin_fabsf(p));
      gate[m] = (p >= 0.0f) ? 1.0f / (1.0f + e) : e / (1.0f + e);
    }
  }
}

// The same computation with x and w staged through LDS (rows 16-byte aligned,
// x and w of one dtype).  A lane reading its own block straight from memory
// touches a different 128-byte line per lane on every load; here each
// wavefront moves 128-byte pieces of all its blocks into a private LDS ring
// with global_load_lds_dwordx4 (eight lanes per line), and each lane reads
// its block's pieces back in order.  The pieces of a wavefront's 64 (row,
// block) slots sit 128 bytes apart, slot q at q * 128; unit i of slot q is
// stored at position i ^ ((q >> 1) & 7) of its eight, so each 16 lanes that
// the LDS serves together reach 16 distinct 16-byte bank groups.  w is copied
// into LDS once per workgroup, unit u of block b at position u ^ (b & 15)
// within the block, for the same reason.  The fmaf order per lane and the
// butterfly are those of the direct kernel above, so both give the same bits.
template <bool B, int LPR>
struct GdLds {
  static constexpr int RPW = 64 / LPR;            // rows per wavefront
  static constexpr int ESZ = B ? 2 : 4;
  static constexpr int PE = 16 / ESZ;             // elements per 16-byte unit
  static constexpr int UPB = 256 / PE;            // units per block (32 or 64)
  static constexpr int CH = 8;                    // units per block per chunk (128 bytes)
  static constexpr int NCH = UPB / CH;            // chunks per block
  static constexpr int UPC = 64 * CH;             // units per chunk and wavefront
  static constexpr int TPC = UPC / 64;            // transfers per chunk (8)
  static constexpr int WU = LPR * UPB;            // units of w held in LDS
  static constexpr int S = (GD_WAVES * 4 * UPC + WU) * 16 <= 160 * 1024 ? 4 : 3;  // ring stages
  static_assert(NCH >= S - 1 && TPC * (S - 1) <= 63, "chunking");
  static_assert((GD_WAVES * S * UPC + WU) * 16 <= 160 * 1024, "LDS");
};

// x is read exactly once.  For fp32 rows its transfers carry the
// non-temporal hint (measured in one process at M = K = 4096: 11.9 us
// against 14.5 us); for bf16 rows the hint measured 3% slower.
__device__ __forceinline__ void dma16_stream(const void *src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds_base) : "memory");
}

template <class C>
__device__ __forceinline__ void gd_issue(const char *__restrict__ x, int64_t M, int K, int64_t mrow0, int nb,
                                         int lane, int c, uint32_t slot) {
#pragma unroll
  for (int t = 0; t < C::TPC; ++t) {
    const int p = 64 * t + lane;                // unit position within the chunk
    const int q = p / C::CH;                    // slot = row * LPR + block
    const int i = (p % C::CH) ^ ((q >> 1) & 7);  // unit of the block's piece held there
    const int rr = q / (64 / C::RPW), bb = q % (64 / C::RPW);
    const int e = 256 * bb + (c * C::CH + i) * C::PE;  // its first element within the row
    const int64_t mm = mrow0 + rr;
    const void *src = &g_pad_pos;
    if (c < C::NCH && mm < M && bb < nb && e < K) src = x + (mm * K + e) * C::ESZ;
    if constexpr (C::ESZ == 4) dma16_stream(src, slot + 1024 * t);
    else dma16(src, slot + 1024 * t);
  }
}

template <bool B, int LPR>
__global__ __launch_bounds__(GD_WAVES * 64) void gate_dot_lds_kernel(const void *__restrict__ x,
                                                                      const void *__restrict__ w,
                                                                      float *__restrict__ dot,
                                                                      float *__restrict__ gate, int64_t M, int K) {
  using C = GdLds<B, LPR>;
  constexpr int S = C::S, PE = C::PE, CH = C::CH;
  __shared__ __attribute__((aligned(16))) uint4 ring[GD_WAVES][S][C::UPC];
  __shared__ __attribute__((aligned(16))) uint4 wl[C::WU];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = lane % LPR, r = lane / LPR;
  const int64_t mrow0 = (static_cast<int64_t>(blockIdx.x) * GD_WAVES + wave) * C::RPW;
  const int64_t m = mrow0 + r;
  const int nb = (K + 255) / 256;
  const char *xc = static_cast<const char *>(x);

  // w into LDS (ordinary loads, completed before the transfers below start)
  const uint4 *wg = static_cast<const uint4 *>(w);
  const int wunits = K / PE;
  for (int u = threadIdx.x; u < wunits; u += GD_WAVES * 64) {
    const int bw = u / C::UPB, iw = u % C::UPB;
    wl[bw * C::UPB + (iw ^ (bw & 15))] = wg[u];
  }
  __syncthreads();

  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<const float *>(ring[wave][0])));
#pragma unroll
  for (int i = 0; i < S - 1; ++i) gd_issue<C>(xc, M, K, mrow0, nb, lane, i, base + i * C::UPC * 16);
  const int cnt = (b < nb) ? min(256, K - 256 * b) : 0;  // elements of this lane's block
  const int sx = (lane >> 1) & 7, sw = b & 15;
  float p = (m < M && b < nb) ? 0.0f : -0.0f;
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    compiler_fence();
    wait_vmcnt<C::TPC * (S - 2)>();
    compiler_fence();
    gd_issue<C>(xc, M, K, mrow0, nb, lane, c + S - 1, base + ((c + S - 1) % S) * C::UPC * 16);
    const uint4 *cur = ring[wave][c % S] + lane * CH;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int u = c * CH + i;  // unit within the block
      if (u * PE < cnt && m < M) {
        float xv[PE], wv[PE];
        unpack16<B>(cur[i ^ sx], xv);
        unpack16<B>(wl[b * C::UPB + (u ^ sw)], wv);
#pragma unroll
        for (int j = 0; j < PE; ++j) p = __builtin_fmaf(xv[j], wv[j], p);
      }
    }
  }
  // no transfer may still be writing LDS when the workgroup exits
  compiler_fence();
  wait_vmcnt<0>();
#pragma unroll
  for (int d = 1; d < LPR; d <<= 1) p = p + __shfl_xor(p, d, 64);
  if (m < M && b == 0) {
    if (dot) dot[m] = p;
    if (gate) {
      const float e = route_exp(-__builtin_fabsf(p));
      gate[m] = (p >= 0.0f) ? 1.0f / (1.0f + e) : e / (1.0f + e);
    }
  }
}

template <bool B, int LPR>
static void launch_gd_lds(const void *x, const void *w, float *dot, float *gate, int64_t M, int K,
                          hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(GD_WAVES) * (64 / LPR);
  const dim3 grid(static_cast<uint32_t>((M + rows_per_block - 1) / rows_per_block)), block(GD_WAVES * 64);
  hipLaunchKernelGGL((gate_dot_lds_kernel<B, LPR>), grid, block, 0, stream, x, w, dot, gate, M, K);
}

template <bool XB, bool WB, int LPR>
static void launch_gd(const void *x, const void *w, float *dot, float *gate, int64_t M, int K, int vec,
                      hipStream_t stream) {
  if constexpr (XB == WB && LPR >= 2) {
    if (vec) return launch_gd_lds<XB, LPR>(x, w, dot, gate, M, K, stream);
  }
  constexpr int RPW = 64 / LPR;
  const int64_t rows_per_block = static_cast<int64_t>(GD_WAVES) * RPW;
  const dim3 grid(static_cast<uint32_t>((M + rows_per_block - 1) / rows_per_block)), block(GD_WAVES * 64);
  hipLaunchKernelGGL((gate_dot_kernel<XB, WB, LPR>), grid, block, 0, stream, x, w, dot, gate, M, K, vec);
}

template <bool XB, bool WB>
static void launch_gd_lpr(const void *x, const void *w, float *dot, float *gate, int64_t M, int K, int vec,
                          hipStream_t stream) {
  const int nb = (K + 255) / 256;
  if (nb <= 1) launch_gd<XB, WB, 1>(x, w, dot, gate, M, K, vec, stream);
  else if (nb <= 2) launch_gd<XB, WB, 2>(x, w, dot, gate, M, K, vec, stream);
  else if (nb <= 4) launch_gd<XB, WB, 4>(x, w, dot, gate, M, K, vec, stream);
  else if (nb <= 8) launch_gd<XB, WB, 8>(x, w, dot, gate, M, K, vec, stream);
  else if (nb <= 16) launch_gd<XB, WB, 16>(x, w, dot, gate, M, K, vec, stream);
  else if (nb <= 32) launch_gd<XB, WB, 32>(x, w, dot, gate, M, K, vec, stream);
  else launch_gd<XB, WB, 64>(x, w, dot, gate, M, K, vec, stream);
}

hipError_t launch_gate_dot(const void *x, int x_bf16, const void *w, int w_bf16, float *dot,
                           float *gate, int64_t M, int64_t K, hipStream_t stream) {
  const int k = static_cast<int>(K);
  // 16-byte pieces need every row (and w) to start 16-byte aligned
  const int vec = ((K * (x_bf16 ? 2 : 4)) % 16 == 0) ? 1 : 0;
  if (x_bf16 && w_bf16) launch_gd_lpr<true, true>(x, w, dot, gate, M, k, vec, stream);
  else if (x_bf16) launch_gd_lpr<true, false>(x, w, dot, gate, M, k, vec, stream);
  else if (w_bf16) launch_gd_lpr<false, true>(x, w, dot, gate, M, k, vec, stream);
  else launch_gd_lpr<false, false>(x, w, dot, gate, M, k, vec, stream);
  return hipGetLastError();
}

}  // namespace drk
