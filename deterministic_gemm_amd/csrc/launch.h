// launch.h -- host-side description of one validated dr_route call, handed
// from the C ABI (dr_api.cpp) to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dr.h"

namespace drk {

struct RouteLaunch {
  const float *xf;     // x as fp32, or NULL
  const uint16_t *xb;  // x as bf16 bits, or NULL
  const float *W;
  int64_t M, K, E;
  int k;
  int logit_bf16;
  uint32_t flags;
  int32_t *ids;
  float *weights;
  void *logits;
  dr_margin *margins;
  hipStream_t stream;
};

hipError_t launch_gemm_bf16_out_bf16(const uint16_t *x, const uint16_t *W, uint16_t *out, int64_t M, int64_t K,
                                     int64_t N, hipStream_t stream);
hipError_t launch_grouped_gemm_bf16(const uint16_t *x, int64_t Mx, const int32_t *rows, const uint16_t *W,
                                    const int32_t *offsets, int64_t E, int64_t P, int64_t K, int64_t N,
                                    float *out, hipStream_t stream);
hipError_t launch_moe_permute(const int32_t *ids, int64_t M, int k, int E, int32_t *offsets, int32_t *rows,
                              int32_t *pos, hipStream_t stream);
hipError_t launch_moe_gather(const void *x, int64_t Mx, int64_t row_bytes, const int32_t *rows, int64_t P,
                             void *xp, hipStream_t stream);
hipError_t launch_moe_combine(const void *y, int y_bf16, int64_t P, const float *weights, const int32_t *ids,
                              const int32_t *pos, const void *shared, int shared_bf16, const float *gate,
                              int64_t M, int k, int64_t D, float *out, hipStream_t stream);

// dr_route_noalloc: the size of the library's static device buffer (the
// logits of 16384 tokens x 256 experts in fp32), and its address on the
// current device (looked up on the first call per device).
constexpr int64_t kNoallocScratchBytes = int64_t(16) << 20;
hipError_t noalloc_scratch(void **ptr);

// Compute units of the current device (256 if the query fails).
int64_t narrow_max_m(int64_t E, int64_t K);
int device_cus();

hipError_t launch_route_rowwise(const RouteLaunch &L);
hipError_t launch_route_tiled(const RouteLaunch &L);
bool tiled_supports(int64_t E, int64_t K);
hipError_t launch_route_split(const RouteLaunch &L);
hipError_t launch_route_fused(const RouteLaunch &L);
bool fused_supports(int64_t E, int64_t K, bool x_f32);
bool split_supports(int64_t E, int64_t K, bool x_f32, bool has_logits);
hipError_t launch_route_tiny(const RouteLaunch &L);
hipError_t launch_route_tiny_logits(const RouteLaunch &L);
bool tiny_supports(int64_t E, int64_t K, bool x_f32, bool has_logits);
hipError_t launch_widen_bf16(const uint16_t *x, int64_t n, float *out, hipStream_t stream);
// the most rows the vector-ALU family's grid takes (four tokens per row of workgroups)
constexpr int64_t kTinyMaxRows = 4 * 65535;
int64_t tiny_max_m(int64_t E, int64_t K);
hipError_t launch_route_narrow(const RouteLaunch &L);
hipError_t launch_route_narrow_logits(const RouteLaunch &L);
bool narrow_supports(int64_t E, int64_t K, bool x_f32, bool has_logits);
// The two halves of the split family on their own.
hipError_t launch_route_logits(const RouteLaunch &L);
hipError_t launch_route_select(const RouteLaunch &L);
bool select_supports(int64_t E);

hipError_t launch_gate_dot(const void *x, int x_bf16, const void *w, int w_bf16, float *dot,
                           float *gate, int64_t M, int64_t K, hipStream_t stream);
hipError_t launch_gemm_bf16(const uint16_t *x, const uint16_t *W, float *out, int64_t M,
                            int64_t K, int64_t N, hipStream_t stream);

}  // namespace drk
