// dr_api.cpp -- the C ABI of include/dr.h: argument validation, the choice
// of kernel family and tile from the shape alone, and the launch on the
// caller's stream.  No numeric decision is made here: every variant computes
// the same canonical order.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/dr.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

dr_status fail(dr_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

dr_status device_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return DR_OK;
  return fail(DR_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxK = 16384;
constexpr int32_t kMaxTopK = 32;
// Rows (tokens) per call.  Every launch keeps its work-items per grid
// dimension below 2^32 up to this bound (the largest is the narrow family at
// E = 512: 2^18 workgroups x 32 expert tiles x 256 lanes).  At K = 2048 it is
// 32 GiB of fp32 activations.
constexpr int64_t kMaxM = int64_t(1) << 22;

// Batches at or above this size run on the matrix-core kernel.  The value sits
// inside the 19..80 token m-scan on purpose, so that scan crosses a dispatch
// change and shows it cannot move a bit.
constexpr int64_t kTiledMinM = 48;
// Calls that ask for the logits run as two kernels, the logits then the
// selection.  Up to drk::narrow_max_m(E, K) tokens the logits spread over
// small (token, expert) tiles with the K groups split between wavefronts;
// above it they use 64 x 64 or 64 x 128 tiles.  Without the logits output the
// fused kernels run.

// noalloc: dr_route_noalloc, which keeps the logits of a two-launch family in
// the library's static device buffer when the caller passes no logits buffer.
dr_status route_impl(const void *x, dr_dtype x_dtype, const float *W, int64_t M, int64_t K,
                     int64_t E, int32_t k, dr_dtype logit_dtype, int32_t *ids, float *weights,
                     void *logits, dr_margin *margins, uint32_t flags, dr_variant variant,
                     void *stream, bool noalloc = false) {
  g_last_error[0] = '\0';
  if (M < 0 || M > kMaxM) return fail(DR_ERR_INVALID, "M=%lld out of range", (long long)M);
  if (K < 1) return fail(DR_ERR_INVALID, "K=%lld must be >= 1", (long long)K);
  if (E < 1) return fail(DR_ERR_INVALID, "E=%lld must be >= 1", (long long)E);
  if (k < 1 || k > E) return fail(DR_ERR_INVALID, "k=%d must be in [1, E=%lld]", k, (long long)E);
  if (x_dtype != DR_F32 && x_dtype != DR_BF16) return fail(DR_ERR_INVALID, "bad x_dtype");
  if (logit_dtype != DR_F32 && logit_dtype != DR_BF16) return fail(DR_ERR_INVALID, "bad logit_dtype");
  if (flags & ~DR_ROUTE_RENORMALIZE) return fail(DR_ERR_INVALID, "unknown flags 0x%x", flags);
  if (variant != DR_VARIANT_AUTO && variant != DR_VARIANT_ROWWISE && variant != DR_VARIANT_TILED &&
      variant != DR_VARIANT_SPLIT && variant != DR_VARIANT_NARROW && variant != DR_VARIANT_TINY &&
      variant != DR_VARIANT_FUSED)
    return fail(DR_ERR_INVALID, "bad variant");
  if (M > 0 && (!x || !W || !ids)) return fail(DR_ERR_INVALID, "x, W and ids are required");
  if (!aligned16(x) || !aligned16(W) || !aligned16(ids) || !aligned16(weights) || !aligned16(logits) ||
      !aligned16(margins))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (!(E == 64 || E == 128 || E == 256 || E == 512 || E == 1024))
    return fail(DR_ERR_UNSUPPORTED, "E=%lld: supported E are 64, 128, 256, 512, 1024", (long long)E);
  if (K > kMaxK) return fail(DR_ERR_UNSUPPORTED, "K=%lld above %lld", (long long)K, (long long)kMaxK);
  if (k > kMaxTopK) return fail(DR_ERR_UNSUPPORTED, "k=%d above %d", k, kMaxTopK);
  if (noalloc && !logits) {
    // the family AUTO picks given a logits buffer; the two-launch ones keep
    // the logits between their launches in the static buffer
    const dr_variant v = dr_route_auto_variant(M, K, E, x_dtype, 1);
    if (v == DR_VARIANT_TINY || v == DR_VARIANT_NARROW || v == DR_VARIANT_SPLIT) {
      const int64_t bytes = M * E * (logit_dtype == DR_BF16 ? 2 : 4);
      if (bytes > drk::kNoallocScratchBytes)
        return fail(DR_ERR_UNSUPPORTED,
                    "dr_route_noalloc: the logits of M=%lld x E=%lld (%lld bytes) exceed its %lld-byte device "
                    "buffer; pass a logits buffer or split the batch",
                    (long long)M, (long long)E, (long long)bytes, (long long)drk::kNoallocScratchBytes);
      if (M == 0) return DR_OK;
      void *buf = nullptr;
      const dr_status s = device_status(drk::noalloc_scratch(&buf), "dr_route_noalloc: device buffer lookup");
      if (s != DR_OK) return s;
      logits = buf;
      variant = v;
    }
  }
  if (variant == DR_VARIANT_AUTO) variant = dr_route_auto_variant(M, K, E, x_dtype, logits != nullptr);
  if (variant == DR_VARIANT_TILED && !drk::tiled_supports(E, K))
    return fail(DR_ERR_UNSUPPORTED, "tiled variant does not support E=%lld", (long long)E);
  if (variant == DR_VARIANT_SPLIT && !drk::split_supports(E, K, x_dtype == DR_F32, logits != nullptr))
    return fail(DR_ERR_UNSUPPORTED,
                "split variant needs E in {256, 512, 1024}, the logits output, and fp32 x with K %% 4 == 0 or bf16 x "
                "with K %% 8 == 0 and K <= 4096");
  if (variant == DR_VARIANT_FUSED && !drk::fused_supports(E, K, x_dtype == DR_F32))
    return fail(DR_ERR_UNSUPPORTED,
                "fused variant needs E = 256 and fp32 x with K %% 4 == 0 or bf16 x with K %% 8 == 0 and K <= 4096");
  if (variant == DR_VARIANT_NARROW && !drk::narrow_supports(E, K, x_dtype == DR_F32, logits != nullptr))
    return fail(DR_ERR_UNSUPPORTED,
                "narrow variant needs E <= 512, the logits output, and K %% 4 == 0 (fp32 x) or K %% 8 == 0 (bf16 x)");
  if (variant == DR_VARIANT_TINY && !drk::tiny_supports(E, K, x_dtype == DR_F32, logits != nullptr))
    return fail(DR_ERR_UNSUPPORTED, "tiny variant needs K %% 4 == 0 (fp32 x) or K %% 8 == 0 (bf16 x), K <= 4096 and the logits output");
  if (variant == DR_VARIANT_TINY && M > drk::kTinyMaxRows)
    return fail(DR_ERR_UNSUPPORTED, "tiny variant takes at most %lld tokens", (long long)drk::kTinyMaxRows);
  if (M == 0) return DR_OK;

  drk::RouteLaunch L;
  L.xf = x_dtype == DR_F32 ? static_cast<const float *>(x) : nullptr;
  L.xb = x_dtype == DR_BF16 ? static_cast<const uint16_t *>(x) : nullptr;
  L.W = W;
  L.M = M;
  L.K = K;
  L.E = E;
  L.k = k;
  L.logit_bf16 = logit_dtype == DR_BF16;
  L.flags = flags;
  L.ids = ids;
  L.weights = weights;
  L.logits = logits;
  L.margins = margins;
  L.stream = static_cast<hipStream_t>(stream);
  const hipError_t e = variant == DR_VARIANT_SPLIT    ? drk::launch_route_split(L)
                       : variant == DR_VARIANT_FUSED  ? drk::launch_route_fused(L)
                       : variant == DR_VARIANT_NARROW ? drk::launch_route_narrow(L)
                       : variant == DR_VARIANT_TINY   ? drk::launch_route_tiny(L)
                       : variant == DR_VARIANT_TILED  ? drk::launch_route_tiled(L)
                                                      : drk::launch_route_rowwise(L);
  return device_status(e, "route launch");
}

}  // namespace

namespace drk {

// The CUs of the current device (the 64 x 128 tiles fill MI355X's 256 at
// M = 8192, E = 256), queried once per device; 256 when no device answers.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace drk

extern "C" {

dr_variant dr_route_auto_variant(int64_t M, int64_t K, int64_t E, dr_dtype x_dtype, int with_logits) {
  // where the narrow family does not take E, the two-kernel family follows
  // the vector-ALU family directly (or takes every batch, past its K)
  const int64_t narrow_max = drk::narrow_supports(E, K, true, true) ? drk::narrow_max_m(E, K)
                             : drk::tiny_supports(E, K, true, true)  ? drk::tiny_max_m(E, K)
                                                                     : 0;
  if (M > narrow_max && drk::split_supports(E, K, x_dtype == DR_F32, with_logits != 0)) return DR_VARIANT_SPLIT;
  if (M <= drk::tiny_max_m(E, K) && drk::tiny_supports(E, K, x_dtype == DR_F32, with_logits != 0)) return DR_VARIANT_TINY;
  if (M <= narrow_max && drk::narrow_supports(E, K, x_dtype == DR_F32, with_logits != 0)) return DR_VARIANT_NARROW;
  if (M >= kTiledMinM && drk::tiled_supports(E, K)) return DR_VARIANT_TILED;
  return DR_VARIANT_ROWWISE;
}

dr_status dr_route(const void *x, dr_dtype x_dtype, const float *W, int64_t M, int64_t K,
                   int64_t E, int32_t k, dr_dtype logit_dtype, int32_t *ids, float *weights,
                   void *logits, dr_margin *margins, uint32_t flags, void *stream) {
  return route_impl(x, x_dtype, W, M, K, E, k, logit_dtype, ids, weights, logits, margins, flags,
                    DR_VARIANT_AUTO, stream);
}

dr_status dr_route_noalloc(const void *x, dr_dtype x_dtype, const float *W, int64_t M, int64_t K,
                           int64_t E, int32_t k, dr_dtype logit_dtype, int32_t *ids, float *weights,
                           void *logits, dr_margin *margins, uint32_t flags, void *stream) {
  return route_impl(x, x_dtype, W, M, K, E, k, logit_dtype, ids, weights, logits, margins, flags,
                    DR_VARIANT_AUTO, stream, true);
}

dr_status dr_route_variant(const void *x, dr_dtype x_dtype, const float *W, int64_t M,
                           int64_t K, int64_t E, int32_t k, dr_dtype logit_dtype, int32_t *ids,
                           float *weights, void *logits, dr_margin *margins, uint32_t flags,
                           dr_variant variant, void *stream) {
  return route_impl(x, x_dtype, W, M, K, E, k, logit_dtype, ids, weights, logits, margins, flags,
                    variant, stream);
}

dr_status dr_route_logits(const float *x, const float *W, int64_t M, int64_t K, int64_t E,
                          dr_dtype logit_dtype, void *logits, void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || M > kMaxM) return fail(DR_ERR_INVALID, "M=%lld out of range", (long long)M);
  if (K < 1) return fail(DR_ERR_INVALID, "K=%lld must be >= 1", (long long)K);
  if (E < 1) return fail(DR_ERR_INVALID, "E=%lld must be >= 1", (long long)E);
  if (logit_dtype != DR_F32 && logit_dtype != DR_BF16) return fail(DR_ERR_INVALID, "bad logit_dtype");
  if (M > 0 && (!x || !W || !logits)) return fail(DR_ERR_INVALID, "x, W and logits are required");
  if (!aligned16(x) || !aligned16(W) || !aligned16(logits))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (!drk::narrow_supports(E, K, true, true))
    return fail(DR_ERR_UNSUPPORTED, "dr_route_logits needs K %% 4 == 0, K <= %lld and E in {64, 128, 256, 512}",
                (long long)kMaxK);
  if (M == 0) return DR_OK;
  drk::RouteLaunch L{};
  L.xf = x;
  L.W = W;
  L.M = M;
  L.K = K;
  L.E = E;
  L.logit_bf16 = logit_dtype == DR_BF16;
  L.logits = logits;
  L.stream = static_cast<hipStream_t>(stream);
  const bool split = M > drk::narrow_max_m(E, K) && drk::split_supports(E, K, true, true);
  const bool tiny = M <= drk::tiny_max_m(E, K) && drk::tiny_supports(E, K, true, true);
  return device_status(split  ? drk::launch_route_logits(L)
                       : tiny ? drk::launch_route_tiny_logits(L)
                              : drk::launch_route_narrow_logits(L),
                       "logits launch");
}

dr_status dr_route_select(const void *logits, dr_dtype logit_dtype, int64_t M, int64_t E, int32_t k,
                          int32_t *ids, float *weights, dr_margin *margins, uint32_t flags,
                          void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || M > kMaxM) return fail(DR_ERR_INVALID, "M=%lld out of range", (long long)M);
  if (E < 1) return fail(DR_ERR_INVALID, "E=%lld must be >= 1", (long long)E);
  if (k < 1 || k > E) return fail(DR_ERR_INVALID, "k=%d must be in [1, E=%lld]", k, (long long)E);
  if (logit_dtype != DR_F32 && logit_dtype != DR_BF16) return fail(DR_ERR_INVALID, "bad logit_dtype");
  if (flags & ~DR_ROUTE_RENORMALIZE) return fail(DR_ERR_INVALID, "unknown flags 0x%x", flags);
  if (M > 0 && (!logits || !ids)) return fail(DR_ERR_INVALID, "logits and ids are required");
  if (!aligned16(logits) || !aligned16(ids) || !aligned16(weights) || !aligned16(margins))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (!drk::select_supports(E))
    return fail(DR_ERR_UNSUPPORTED, "E=%lld: dr_route_select supports E in {64, 128, 256, 512, 1024}",
                (long long)E);
  if (k > kMaxTopK) return fail(DR_ERR_UNSUPPORTED, "k=%d above %d", k, kMaxTopK);
  if (M == 0) return DR_OK;
  drk::RouteLaunch L{};
  L.M = M;
  L.E = E;
  L.k = k;
  L.logit_bf16 = logit_dtype == DR_BF16;
  L.flags = flags;
  L.ids = ids;
  L.weights = weights;
  L.logits = const_cast<void *>(logits);
  L.margins = margins;
  L.stream = static_cast<hipStream_t>(stream);
  return device_status(drk::launch_route_select(L), "select launch");
}

dr_status dr_gate_dot(const void *x, dr_dtype x_dtype, const void *w, dr_dtype w_dtype,
                      float *dot, float *gate, int64_t M, int64_t K, void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || M > kMaxM) return fail(DR_ERR_INVALID, "M=%lld out of range", (long long)M);
  if (K < 1) return fail(DR_ERR_INVALID, "K=%lld must be >= 1", (long long)K);
  if ((x_dtype != DR_F32 && x_dtype != DR_BF16) || (w_dtype != DR_F32 && w_dtype != DR_BF16))
    return fail(DR_ERR_INVALID, "bad dtype");
  if (M > 0 && (!x || !w)) return fail(DR_ERR_INVALID, "x and w are required");
  if (M > 0 && !dot && !gate) return fail(DR_ERR_INVALID, "one of dot, gate is required");
  if (!aligned16(x) || !aligned16(w) || !aligned16(dot) || !aligned16(gate))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (K > kMaxK) return fail(DR_ERR_UNSUPPORTED, "K=%lld above %lld", (long long)K, (long long)kMaxK);
  if (M == 0) return DR_OK;
  return device_status(drk::launch_gate_dot(x, x_dtype == DR_BF16, w, w_dtype == DR_BF16, dot, gate, M, K,
                                            static_cast<hipStream_t>(stream)),
                       "gate_dot launch");
}

dr_status dr_gemm_bf16(const uint16_t *x, const uint16_t *W, float *out, int64_t M, int64_t K,
                       int64_t N, void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || K < 1 || N < 1) return fail(DR_ERR_INVALID, "bad sizes");
  if (M > 0 && (!x || !W || !out)) return fail(DR_ERR_INVALID, "x, W and out are required");
  if (!aligned16(x) || !aligned16(W) || !aligned16(out))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (K % 32 != 0 || N % 128 != 0)
    return fail(DR_ERR_UNSUPPORTED, "K must be a multiple of 32 and N of 128");
  if (K > (int64_t(1) << 30) || N > (int64_t(1) << 30) || M > int64_t(65535) * 128)
    return fail(DR_ERR_UNSUPPORTED, "size out of range");
  if (M == 0) return DR_OK;
  return device_status(drk::launch_gemm_bf16(x, W, out, M, K, N, static_cast<hipStream_t>(stream)),
                       "gemm launch");
}

dr_status dr_route_bf16_gemm(const uint16_t *x, const uint16_t *W, int64_t M, int64_t K, int64_t E,
                             int32_t k, int32_t *ids, float *weights, uint16_t *logits, dr_margin *margins,
                             uint32_t flags, void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || M > kMaxM) return fail(DR_ERR_INVALID, "M=%lld out of range", (long long)M);
  if (K < 1 || E < 1) return fail(DR_ERR_INVALID, "bad sizes");
  if (k < 1 || k > E) return fail(DR_ERR_INVALID, "k=%d must be in [1, E=%lld]", k, (long long)E);
  if (flags & ~DR_ROUTE_RENORMALIZE) return fail(DR_ERR_INVALID, "unknown flags 0x%x", flags);
  if (M > 0 && (!x || !W || !ids || !logits)) return fail(DR_ERR_INVALID, "x, W, ids and logits are required");
  if (!aligned16(x) || !aligned16(W) || !aligned16(ids) || !aligned16(weights) || !aligned16(logits) ||
      !aligned16(margins))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (K % 32 != 0 || E % 128 != 0 || !drk::select_supports(E) || K > (int64_t(1) << 30))
    return fail(DR_ERR_UNSUPPORTED, "dr_route_bf16_gemm needs K %% 32 == 0 and E in {128, 256, 512, 1024}");
  if (k > kMaxTopK) return fail(DR_ERR_UNSUPPORTED, "k=%d above %d", k, kMaxTopK);
  if (M == 0) return DR_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dr_status s1 = device_status(drk::launch_gemm_bf16_out_bf16(x, W, logits, M, K, E, st), "gate gemm launch");
  if (s1 != DR_OK) return s1;
  drk::RouteLaunch L{};
  L.M = M;
  L.E = E;
  L.k = k;
  L.logit_bf16 = 1;
  L.flags = flags;
  L.ids = ids;
  L.weights = weights;
  L.logits = logits;
  L.margins = margins;
  L.stream = st;
  return device_status(drk::launch_route_select(L), "select launch");
}

dr_status dr_grouped_gemm_bf16(const uint16_t *x, int64_t Mx, const int32_t *rows, const uint16_t *W,
                               const int32_t *offsets, int64_t E, int64_t P, int64_t K, int64_t N,
                               float *out, void *stream) {
  g_last_error[0] = '\0';
  if (Mx < 0 || P < 0 || K < 1 || N < 1 || E < 1) return fail(DR_ERR_INVALID, "bad sizes");
  if (!offsets || (P > 0 && (!x || !W || !out))) return fail(DR_ERR_INVALID, "x, W, offsets and out are required");
  if (!rows && P > Mx) return fail(DR_ERR_INVALID, "without rows, x must hold the P grouped rows");
  if (!aligned16(x) || !aligned16(rows) || !aligned16(W) || !aligned16(offsets) || !aligned16(out))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (K % 32 != 0 || N % 128 != 0) return fail(DR_ERR_UNSUPPORTED, "K must be a multiple of 32 and N of 128");
  if (E > 1024 || P > INT32_MAX || Mx > INT32_MAX || K > (int64_t(1) << 30) || N > (int64_t(1) << 30) ||
      (P + 127) / 128 + E > 65535 || 8 * (((P + 127) / 128 + E + 7) / 8) * (N / 128) > int64_t(UINT32_MAX))
    return fail(DR_ERR_UNSUPPORTED, "size out of range");
  if (P == 0) return DR_OK;
  return device_status(drk::launch_grouped_gemm_bf16(x, Mx, rows, W, offsets, E, P, K, N, out,
                                                     static_cast<hipStream_t>(stream)),
                       "grouped gemm launch");
}

dr_status dr_moe_permute(const int32_t *ids, int64_t M, int32_t k, int32_t E, int32_t *offsets,
                         int32_t *rows, int32_t *pos, void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || k < 1 || E < 1 || M > kMaxM) return fail(DR_ERR_INVALID, "bad sizes");
  if (!offsets || (M > 0 && (!ids || !rows || !pos))) return fail(DR_ERR_INVALID, "ids, offsets, rows and pos are required");
  if (!aligned16(ids) || !aligned16(offsets) || !aligned16(rows) || !aligned16(pos))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (k > 32 || E > 1024 || M > INT32_MAX / k)
    return fail(DR_ERR_UNSUPPORTED, "dr_moe_permute needs k <= 32, E <= 1024 and M*k < 2^31");
  return device_status(drk::launch_moe_permute(ids, M, k, E, offsets, rows, pos, static_cast<hipStream_t>(stream)),
                       "moe_permute launch");
}

dr_status dr_moe_gather(const void *x, dr_dtype dtype, int64_t M, int64_t D, const int32_t *rows,
                        int64_t P, void *xp, void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || D < 1 || P < 0) return fail(DR_ERR_INVALID, "bad sizes");
  if (dtype != DR_F32 && dtype != DR_BF16) return fail(DR_ERR_INVALID, "bad dtype");
  if (P > 0 && (!x || !rows || !xp)) return fail(DR_ERR_INVALID, "x, rows and xp are required");
  if (!aligned16(x) || !aligned16(rows) || !aligned16(xp)) return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (P > INT32_MAX || M > INT32_MAX) return fail(DR_ERR_UNSUPPORTED, "P and M must be below 2^31");
  if (P == 0) return DR_OK;
  return device_status(drk::launch_moe_gather(x, M, D * (dtype == DR_BF16 ? 2 : 4), rows, P, xp,
                                              static_cast<hipStream_t>(stream)),
                       "moe_gather launch");
}

dr_status dr_moe_combine(const void *y, dr_dtype y_dtype, int64_t P, const float *weights,
                         const int32_t *ids, const int32_t *pos, const void *shared,
                         dr_dtype shared_dtype, const float *gate, int64_t M, int32_t k, int64_t D,
                         float *out, void *stream) {
  g_last_error[0] = '\0';
  if (M < 0 || k < 1 || D < 1 || P < 0 || (M > 0 && P < 1)) return fail(DR_ERR_INVALID, "bad sizes");
  if (y_dtype != DR_F32 && y_dtype != DR_BF16) return fail(DR_ERR_INVALID, "bad y_dtype");
  if (shared && shared_dtype != DR_F32 && shared_dtype != DR_BF16) return fail(DR_ERR_INVALID, "bad shared_dtype");
  if (M > 0 && (!y || !weights || !ids || !pos || !out)) return fail(DR_ERR_INVALID, "y, weights, ids, pos and out are required");
  if (shared && !gate) return fail(DR_ERR_INVALID, "gate is required with shared");
  if (!aligned16(y) || !aligned16(weights) || !aligned16(ids) || !aligned16(pos) || !aligned16(shared) ||
      !aligned16(gate) || !aligned16(out))
    return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (k > 32 || M > kMaxM) return fail(DR_ERR_UNSUPPORTED, "dr_moe_combine needs k <= 32 and M <= 2^22");
  if (M == 0) return DR_OK;
  return device_status(drk::launch_moe_combine(y, y_dtype == DR_BF16, P, weights, ids, pos, shared,
                                               shared && shared_dtype == DR_BF16, gate, M, k, D, out,
                                               static_cast<hipStream_t>(stream)),
                       "moe_combine launch");
}

dr_status dr_widen_bf16(const uint16_t *x, int64_t n, float *out, void *stream) {
  g_last_error[0] = '\0';
  if (n < 0) return fail(DR_ERR_INVALID, "n=%lld must be >= 0", (long long)n);
  if (n > 0 && (!x || !out)) return fail(DR_ERR_INVALID, "x and out are required");
  if (!aligned16(x) || !aligned16(out)) return fail(DR_ERR_INVALID, "pointers must be 16-byte aligned");
  if (n == 0) return DR_OK;
  return device_status(drk::launch_widen_bf16(x, n, out, static_cast<hipStream_t>(stream)), "widen launch");
}

void dr_contract(dr_contract_info *out) {
  if (!out) return;
  out->version = 1;
  out->kblock = 256;
  out->tree = 1;
  out->acc_bits = 32;
  out->fma = 1;
  out->exp_id = 1;
  out->tie_break = 1;
  out->max_k = kMaxTopK;
}

const char *dr_status_string(dr_status s) {
  switch (s) {
    case DR_OK: return "ok";
    case DR_ERR_INVALID: return "invalid argument";
    case DR_ERR_UNSUPPORTED: return "unsupported shape";
    case DR_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char *dr_last_error(void) { return g_last_error; }

}  // extern "C"
