// moe.hip -- the step after routing: grouping a route's assignments by
// expert, copying activation rows into that grouped order, and the MoE
// combine.
//
// vllm.cpp PR #2556 (section "Why a value tap could never have said this")
// describes the engine's MoE combine as order-invariant over a token's k
// slots and names the assembled per-slot expert outputs as one of the MoE
// block's axes.  The readings taken where the pages stop:
//  * grouping: experts ascending; inside an expert, tokens ascending (the
//    stable grouping of the assignments in token order), so the grouped
//    layout is a function of the ids alone;
//  * combine: a token's slots in ascending expert id, one fp32 fmaf chain
//    from +0 per output element, then the gated shared expert as one more
//    fmaf.  Slot order cannot change a bit, and neither can the batch: each
//    token reads only its own slots.
//
// Integer counting in LDS uses atomic adds and ors.  Their results (counts,
// bit sets) do not depend on the order in which lanes arrive, so they keep
// the outputs deterministic; no floating-point value is ever accumulated by
// an atomic.
#include "route_common.h"
#include "launch.h"

namespace drk {

// ------------------------------------------------------------ permutation

constexpr int PERM_T = 512;          // tokens (threads) per workgroup
constexpr int PERM_EMAX = 1024;      // largest expert count
constexpr int PERM_W = PERM_T / 32;  // presence-bit words per expert
constexpr int PERM_U = 8;            // id loads in flight per thread
static_assert(PERM_EMAX <= 2 * PERM_T, "two experts per thread in the scan");

// Each workgroup places the assignments of PERM_T consecutive tokens.  It
// needs, per expert e, the number of assignments to experts < e (the start
// of e's rows) and the number of assignments to e by tokens before its chunk;
// both come from histograms over the whole id array, which each workgroup
// builds itself (the ids are small and L2-resident, and no workspace or
// second launch is needed).  Inside the chunk, a token's rank among the
// chunk's tokens choosing e is the number of set presence bits of e below its
// own: a per-expert running count over whole 32-bit words (built once) plus a
// popcount within the token's word.  Ids outside [0,E) are skipped (their pos
// is -1).  A row that repeats an expert is outside the contract; its
// positions stay inside the expert's range but may coincide.
// The part both permutation paths share, run by a workgroup of PERM_T lanes
// once tot[e] (all assignments to e) and base[e] (assignments to e by tokens
// before the chunk) are in LDS: presence bits of the chunk's tokens, their
// per-word running counts, the exclusive scan of tot (start of each expert's
// rows; workgroup 0 writes offsets), and pos for the chunk's assignments.
__device__ void permute_place(const int32_t *__restrict__ ids, int64_t M, int k, int E, int64_t c0,
                              int32_t *__restrict__ offsets, int32_t *__restrict__ pos, int32_t *tot, int32_t *base,
                              uint32_t *bits, uint16_t *below, int32_t *wsum) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < E * PERM_W; i += PERM_T) bits[i] = 0;
  __syncthreads();
  const int64_t m = c0 + t;
  if (m < M)
    for (int j = 0; j < k; ++j) {
      const int32_t e = ids[m * k + j];
      if (e >= 0 && e < E) atomicOr(&bits[e * PERM_W + t / 32], 1u << (t % 32));
    }
  __syncthreads();

  // running counts of presence bits per expert over whole words
  for (int e = t; e < E; e += PERM_T) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < PERM_W; ++w) {
      below[e * PERM_W + w] = static_cast<uint16_t>(run);
      run += __builtin_popcount(bits[e * PERM_W + w]);
    }
  }
  // exclusive scan of tot over experts: thread t holds experts 2t and 2t+1
  const int e0 = 2 * t, e1 = 2 * t + 1;
  const int c_0 = (e0 < E) ? tot[e0] : 0, c_1 = (e1 < E) ? tot[e1] : 0;
  int v = c_0 + c_1;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int s = (lane < PERM_T / 64) ? wsum[lane] : 0;
#pragma unroll
    for (int d = 1; d < PERM_T / 64; d <<= 1) {
      const int o = __shfl_up(s, d, 64);
      if (lane >= d) s += o;
    }
    if (lane < PERM_T / 64) wsum[lane] = s;
  }
  __syncthreads();
  const int incl = v + (wave > 0 ? wsum[wave - 1] : 0);  // through expert 2t+1
  const int start0 = incl - c_0 - c_1, start1 = incl - c_1;
  if (e0 < E) base[e0] += start0;
  if (e1 < E) base[e1] += start1;
  if (blockIdx.x == 0) {
    if (e0 < E) offsets[e0] = start0;
    if (e1 < E) offsets[e1] = start1;
    if (e0 == E - 1) offsets[E] = start0 + c_0;
    if (e1 == E - 1) offsets[E] = incl;
  }
  __syncthreads();

  if (m < M)
    for (int j = 0; j < k; ++j) {
      const int32_t e = ids[m * k + j];
      if (e < 0 || e >= E) {
        pos[m * k + j] = -1;
        continue;
      }
      const int w = t / 32;
      const int r = below[e * PERM_W + w] + __builtin_popcount(bits[e * PERM_W + w] & ((1u << (t % 32)) - 1u));
      pos[m * k + j] = base[e] + r;
    }
}

__global__ __launch_bounds__(PERM_T) void moe_permute_kernel(const int32_t *__restrict__ ids, int64_t M, int k,
                                                             int E, int vec, int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ rows,
                                                             int32_t *__restrict__ pos) {
  __shared__ int32_t tot[PERM_EMAX];
  __shared__ int32_t base[PERM_EMAX];
  __shared__ uint32_t bits[PERM_EMAX * PERM_W];
  __shared__ uint16_t below[PERM_EMAX * PERM_W];  // set bits of e in words < w
  __shared__ int32_t wsum[PERM_T / 64];
  const int t = threadIdx.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * PERM_T;
  for (int e = t; e < E; e += PERM_T) tot[e] = 0, base[e] = 0;
  __syncthreads();

  // histograms: all assignments (tot) and those of earlier tokens (base)
  const int64_t n = M * k, nbefore = c0 * k;
  auto count = [&](int32_t e, int64_t i) {
    if (e >= 0 && e < E) {
      atomicAdd(&tot[e], 1);
      if (i < nbefore) atomicAdd(&base[e], 1);
    }
  };
  if (vec) {
    const int4 *v = reinterpret_cast<const int4 *>(ids);
    const int64_t nq = n / 4;
    for (int64_t q0 = 0; q0 < nq; q0 += static_cast<int64_t>(PERM_T) * PERM_U) {
      int4 a[PERM_U];
#pragma unroll
      for (int u = 0; u < PERM_U; ++u) {
        const int64_t q = q0 + u * PERM_T + t;
        a[u] = (q < nq) ? v[q] : int4{-1, -1, -1, -1};
      }
#pragma unroll
      for (int u = 0; u < PERM_U; ++u) {
        const int64_t i = 4 * (q0 + u * PERM_T + t);
        count(a[u].x, i);
        count(a[u].y, i + 1);
        count(a[u].z, i + 2);
        count(a[u].w, i + 3);
      }
    }
  } else {
    for (int64_t i0 = 0; i0 < n; i0 += static_cast<int64_t>(PERM_T) * PERM_U) {
      int32_t a[PERM_U];
#pragma unroll
      for (int u = 0; u < PERM_U; ++u) {
        const int64_t i = i0 + u * PERM_T + t;
        a[u] = (i < n) ? ids[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < PERM_U; ++u) count(a[u], i0 + u * PERM_T + t);
    }
  }
  __syncthreads();
  permute_place(ids, M, k, E, c0, offsets, pos, tot, base, bits, below, wsum);
  const int64_t m = c0 + threadIdx.x;
  if (m < M)
    for (int j = 0; j < k; ++j) {
      const int32_t p = pos[m * k + j];
      if (p >= 0) rows[p] = static_cast<int32_t>(m);
    }
}

// The linear path for batches of several chunks, in three launches; the
// first keeps the per-chunk histograms in the caller's rows buffer, which the
// second reads and the third overwrites with the grouped rows' tokens.
__global__ __launch_bounds__(PERM_T) void moe_chunk_hist_kernel(const int32_t *__restrict__ ids, int64_t M, int k,
                                                                int E, int32_t *__restrict__ hist) {
  __shared__ int32_t h[PERM_EMAX];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += PERM_T) h[e] = 0;
  __syncthreads();
  const int64_t m = static_cast<int64_t>(blockIdx.x) * PERM_T + t;
  if (m < M)
    for (int j = 0; j < k; ++j) {
      const int32_t e = ids[m * k + j];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  __syncthreads();
  for (int e = t; e < E; e += PERM_T) hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

__global__ __launch_bounds__(PERM_T) void moe_chunk_place_kernel(const int32_t *__restrict__ ids, int64_t M, int k,
                                                                 int E, int64_t nchunks,
                                                                 const int32_t *__restrict__ hist,
                                                                 int32_t *__restrict__ offsets,
                                                                 int32_t *__restrict__ pos) {
  __shared__ int32_t tot[PERM_EMAX];
  __shared__ int32_t base[PERM_EMAX];
  __shared__ uint32_t bits[PERM_EMAX * PERM_W];
  __shared__ uint16_t below[PERM_EMAX * PERM_W];
  __shared__ int32_t wsum[PERM_T / 64];
  const int t = threadIdx.x;
  const int64_t c = blockIdx.x;
  for (int e = t; e < E; e += PERM_T) {
    int before = 0, all = 0;
    for (int64_t q0 = 0; q0 < nchunks; q0 += PERM_U) {
      int h[PERM_U];
#pragma unroll
      for (int u = 0; u < PERM_U; ++u) h[u] = (q0 + u < nchunks) ? hist[(q0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < PERM_U; ++u) {
        all += h[u];
        before += (q0 + u < c) ? h[u] : 0;
      }
    }
    tot[e] = all, base[e] = before;
  }
  __syncthreads();
  permute_place(ids, M, k, E, c * PERM_T, offsets, pos, tot, base, bits, below, wsum);
}

__global__ __launch_bounds__(256) void moe_scatter_rows_kernel(const int32_t *__restrict__ pos, int64_t n, int k,
                                                               int32_t *__restrict__ rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) {
    const int32_t p = pos[i];
    if (p >= 0) rows[p] = static_cast<int32_t>(i / k);
  }
}

hipError_t launch_moe_permute(const int32_t *ids, int64_t M, int k, int E, int32_t *offsets, int32_t *rows,
                              int32_t *pos, hipStream_t stream) {
  const int64_t nchunks = M > 0 ? (M + PERM_T - 1) / PERM_T : 1;
  if (nchunks >= 2 && nchunks * E <= M * k) {
    const dim3 grid(static_cast<uint32_t>(nchunks));
    hipLaunchKernelGGL(moe_chunk_hist_kernel, grid, dim3(PERM_T), 0, stream, ids, M, k, E, rows);
    hipLaunchKernelGGL(moe_chunk_place_kernel, grid, dim3(PERM_T), 0, stream, ids, M, k, E, nchunks,
                       static_cast<const int32_t *>(rows), offsets, pos);
    const int64_t n = M * k;
    hipLaunchKernelGGL(moe_scatter_rows_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const int32_t *>(pos), n, k, rows);
    return hipGetLastError();
  }
  const int vec = ((M * k) % 4 == 0 && (reinterpret_cast<uintptr_t>(ids) % 16) == 0) ? 1 : 0;
  hipLaunchKernelGGL(moe_permute_kernel, dim3(static_cast<uint32_t>(nchunks)), dim3(PERM_T), 0, stream, ids, M, k,
                     E, vec, offsets, rows, pos);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gather

// One workgroup per grouped row, the grid striding over rows past 65536:
// xp[p] = x[rows[p]] (a row index outside [0, Mx) gives a zero row), in
// 16-byte pieces when rows allow it.
__global__ __launch_bounds__(256) void moe_gather_kernel(const char *__restrict__ x, int64_t Mx,
                                                         const int32_t *__restrict__ rows, int64_t P,
                                                         int64_t row_bytes, char *__restrict__ xp) {
  for (int64_t p = blockIdx.x; p < P; p += gridDim.x) {
    const int32_t r = rows[p];
    const bool ok = r >= 0 && r < Mx;
    const int t = threadIdx.x;
    if (row_bytes % 16 == 0) {
      const uint4 *src = reinterpret_cast<const uint4 *>(x + static_cast<int64_t>(ok ? r : 0) * row_bytes);
      uint4 *dst = reinterpret_cast<uint4 *>(xp + p * row_bytes);
      for (int64_t i = t; i < row_bytes / 16; i += 256) dst[i] = ok ? src[i] : uint4{0u, 0u, 0u, 0u};
    } else {
      const uint16_t *src = reinterpret_cast<const uint16_t *>(x + static_cast<int64_t>(ok ? r : 0) * row_bytes);
      uint16_t *dst = reinterpret_cast<uint16_t *>(xp + p * row_bytes);
      for (int64_t i = t; i < row_bytes / 2; i += 256) dst[i] = ok ? src[i] : static_cast<uint16_t>(0);
    }
  }
}

hipError_t launch_moe_gather(const void *x, int64_t Mx, int64_t row_bytes, const int32_t *rows, int64_t P,
                             void *xp, hipStream_t stream) {
  const int64_t blocks = P < 65536 ? P : 65536;
  hipLaunchKernelGGL(moe_gather_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<const char *>(x), Mx, rows, P, row_bytes, static_cast<char *>(xp));
  return hipGetLastError();
}

// ----------------------------------------------------------------- combine

// Load N consecutive elements (bf16 widened exactly, or f32) starting at
// element i of a row; N * element size is 8, 16 or 32 bytes, and i is a
// multiple of N, so the loads are aligned.
template <bool B, int N>
__device__ __forceinline__ void load_n(const void *p, int64_t i, float (&v)[N]) {
  if constexpr (B) {
    if constexpr (N == 8) {
      const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) v[2 * j] = u2f(w[j] << 16), v[2 * j + 1] = u2f(w[j] & 0xFFFF0000u);
    } else {
      const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
      v[0] = u2f(u.x << 16), v[1] = u2f(u.x & 0xFFFF0000u), v[2] = u2f(u.y << 16), v[3] = u2f(u.y & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i + j);
      v[j] = f.x, v[j + 1] = f.y, v[j + 2] = f.z, v[j + 3] = f.w;
    }
  }
}

// 16 bytes of a row that is read once (the expert outputs), without keeping
// them in the caches: 8 bf16 widened exactly, or 4 fp32.
template <bool B>
__device__ __forceinline__ void load_stream16(const void *p, int64_t i, float (&v)[B ? 8 : 4]) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (B) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + i));
#pragma unroll
    for (int j = 0; j < 4; ++j) v[2 * j] = u2f(u[j] << 16), v[2 * j + 1] = u2f(u[j] & 0xFFFF0000u);
  } else {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(static_cast<const float *>(p) + i));
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = u2f(u[j]);
  }
}

template <bool B>
__device__ __forceinline__ float load_1(const void *p, int64_t i) {
  if constexpr (B) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

constexpr int COMB_WAVES = 4;  // wavefronts per token
constexpr int COMB_KMAX = 32;
constexpr int COMB_U = 8;      // slot loads in flight per lane

// One workgroup of COMB_WAVES wavefronts per token, no workgroup barrier:
// each wavefront sorts the token's slots itself (lane s < k holds slot s and
// counts the slots that precede it in (expert id, slot index) order; that
// rank is where its weight and grouped row go in the wavefront's LDS list),
// then runs the chains of its columns over the sorted list with up to COMB_U
// slots' loads (and the shared row's) in flight before the chains advance.
// A lane takes 16 bytes of each slot's row per pass (8 bf16 or 4 fp32
// columns); the rows, read once, and the output, written once, bypass the
// caches (non-temporal accesses), which measured 64.6 us against 81 us at
// M = 8192, D = 2048, k = 8 with bf16 rows.
// A slot whose grouped row is outside [0,P) is left out (outside the
// contract; no read leaves y).
template <bool YB, bool SB, bool VEC>
__global__ __launch_bounds__(COMB_WAVES * 64) void moe_combine_kernel(const void *__restrict__ y, int64_t P,
                                                                      const float *__restrict__ weights,
                                                                      const int32_t *__restrict__ ids,
                                                                      const int32_t *__restrict__ pos,
                                                                      const void *__restrict__ shared,
                                                                      const float *__restrict__ gate, int64_t M,
                                                                      int k, int64_t D, float *__restrict__ out) {
  __shared__ float sw_all[COMB_WAVES][COMB_KMAX];
  __shared__ int32_t sp_all[COMB_WAVES][COMB_KMAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m = blockIdx.x;
  float *sw = sw_all[wave];
  int32_t *sp = sp_all[wave];
  int32_t e = 0x7FFFFFFF, p = -1;
  float wv = 0.0f;
  if (lane < k) {
    e = ids[m * k + lane];
    wv = weights[m * k + lane];
    const int32_t q = pos[m * k + lane];
    p = (q >= 0 && q < P) ? q : -1;
  }
  int r = 0;
  for (int j = 0; j < k; ++j) {
    const int32_t f = __shfl(e, j, 64);
    r += (f < e || (f == e && j < lane)) ? 1 : 0;
  }
  if (lane < k) sw[r] = wv, sp[r] = p;
  // LDS accesses of one wavefront complete in order; keep the compiler from
  // moving the reads below above these writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float g = shared ? gate[m] : 0.0f;
  const int col = wave * 64 + lane;  // this lane's first column group

  if constexpr (VEC) {
    constexpr int PE = YB ? 8 : 4;  // columns per lane and pass: 16 bytes of each row
    for (int64_t d0 = static_cast<int64_t>(col) * PE; d0 < D; d0 += COMB_WAVES * 64 * PE) {
      float acc[PE], sv[PE];
#pragma unroll
      for (int i = 0; i < PE; ++i) acc[i] = 0.0f;
      if (shared) load_n<SB, PE>(shared, m * D + d0, sv);
      for (int s0 = 0; s0 < k; s0 += COMB_U) {
        float v[COMB_U][PE];
#pragma unroll
        for (int q = 0; q < COMB_U; ++q)
          if (s0 + q < k && sp[s0 + q] >= 0) load_stream16<YB>(y, static_cast<int64_t>(sp[s0 + q]) * D + d0, v[q]);
#pragma unroll
        for (int q = 0; q < COMB_U; ++q)
          if (s0 + q < k && sp[s0 + q] >= 0) {
            const float wq = sw[s0 + q];
#pragma unroll
            for (int i = 0; i < PE; ++i) acc[i] = __builtin_fmaf(wq, v[q][i], acc[i]);
          }
      }
      if (shared) {
#pragma unroll
        for (int i = 0; i < PE; ++i) acc[i] = __builtin_fmaf(g, sv[i], acc[i]);
      }
      typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int i = 0; i < PE; i += 4)
        __builtin_nontemporal_store(f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]},
                                    reinterpret_cast<f32x4 *>(out + m * D + d0 + i));
    }
  } else {
    for (int64_t d = col; d < D; d += COMB_WAVES * 64) {
      float acc = 0.0f;
      for (int s = 0; s < k; ++s)
        if (sp[s] >= 0) acc = __builtin_fmaf(sw[s], load_1<YB>(y, static_cast<int64_t>(sp[s]) * D + d), acc);
      if (shared) acc = __builtin_fmaf(g, load_1<SB>(shared, m * D + d), acc);
      out[m * D + d] = acc;
    }
  }
}

template <bool YB, bool SB>
static void launch_combine_t(const void *y, int64_t P, const float *weights, const int32_t *ids,
                             const int32_t *pos, const void *shared, const float *gate, int64_t M, int k,
                             int64_t D, float *out, hipStream_t stream) {
  const bool vec = D % (YB ? 8 : 4) == 0;
  const dim3 grid(static_cast<uint32_t>(M)), block(COMB_WAVES * 64);
  if (vec)
    hipLaunchKernelGGL((moe_combine_kernel<YB, SB, true>), grid, block, 0, stream, y, P, weights, ids, pos, shared,
                       gate, M, k, D, out);
  else
    hipLaunchKernelGGL((moe_combine_kernel<YB, SB, false>), grid, block, 0, stream, y, P, weights, ids, pos, shared,
                       gate, M, k, D, out);
}

hipError_t launch_moe_combine(const void *y, int y_bf16, int64_t P, const float *weights, const int32_t *ids,
                              const int32_t *pos, const void *shared, int shared_bf16, const float *gate,
                              int64_t M, int k, int64_t D, float *out, hipStream_t stream) {
  if (y_bf16 && shared_bf16) launch_combine_t<true, true>(y, P, weights, ids, pos, shared, gate, M, k, D, out, stream);
  else if (y_bf16) launch_combine_t<true, false>(y, P, weights, ids, pos, shared, gate, M, k, D, out, stream);
  else if (shared_bf16) launch_combine_t<false, true>(y, P, weights, ids, pos, shared, gate, M, k, D, out, stream);
  else launch_combine_t<false, false>(y, P, weights, ids, pos, shared, gate, M, k, D, out, stream);
  return hipGetLastError();
}

}  // namespace drk
