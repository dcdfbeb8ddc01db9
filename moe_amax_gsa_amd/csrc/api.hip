// api.hip -- the C ABI declared in include/nvfp4.h: argument validation,
// workspace sizing and dispatch to the gfx950 kernels.  Nothing here touches
// device memory from the host; every launch goes to the caller's stream.
#include <stdint.h>

#include "../../include/nvfp4.h"
#include "launch.hpp"

#define NVFP4_API extern "C" __attribute__((visibility("default")))

using namespace nvfp4;

namespace {

constexpr int64_t I32_MAX = 2147483647;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool dtype_ok(int d) { return d == NVFP4_DTYPE_BF16 || d == NVFP4_DTYPE_FP32; }
inline int launched(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH; }

size_t amax_ws_bytes(int64_t numel) {
  if (numel <= AMAX_SMALL_NUMEL) return 0;
  return (size_t)amax_parts_for(numel) * sizeof(uint32_t);
}

// Shape checks shared by the linear entry points.
int check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (M > I32_MAX || N > I32_MAX || K > I32_MAX) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

}  // namespace

NVFP4_API int nvfp4_abi_version(void) { return 10; }

NVFP4_API const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "unsupported shape (negative size, K <= 0 or K % 16 != 0, or too large)";
    case NVFP4_ERR_DTYPE: return "unknown dtype";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_ALIGN: return "pointer not aligned as required";
    case NVFP4_ERR_LAUNCH: return "HIP launch failed";
    case NVFP4_ERR_SCRATCH:
      return "the call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

// split-K partials of the tiled kernel (shapes with few output tiles)
static size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return (M > GEMV_MAX_M && N > 0 && K > 0) ? gemm_ws_bytes(M, N, K) : 0;
}

static size_t round16(size_t n) { return (n + 15) & ~(size_t)15; }

// workspace of the grouped run (the amax partials, past the one-launch size;
// the fallback path's amax partials are never more) and of the MoE run
static size_t grouped_run_ws_bytes_any(int64_t rows, int64_t K);
static size_t moe_ws_bytes_any(int64_t T, int64_t N1, int64_t K1, int E);

NVFP4_API size_t nvfp4_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int G) {
  (void)N;
  (void)K;
  (void)G;
  switch (op) {
    case NVFP4_OP_AMAX_GSA: return M > 0 ? amax_ws_bytes(M) : 0;
    case NVFP4_OP_LINEAR: return linear_ws_bytes(M, N, K);
    case NVFP4_OP_LINEAR_RUN: {
      const size_t a = (M > 0 && K > 0) ? amax_ws_bytes(M * K) : 0;
      const size_t l = linear_ws_bytes(M, N, K);
      return a > l ? a : l;
    }
    case NVFP4_OP_QUANTIZE_WEIGHT: return (N > 0 && K > 0) ? amax_ws_bytes(N * K) : 0;
    case NVFP4_OP_RMSNORM_QUANTIZE: return M > 0 ? (size_t)M * sizeof(uint32_t) : 0;
    case NVFP4_OP_ROUTER_TOPK:
      // the logits, then the one-launch path's ticket counter (M <= 16) or
      // the linear's split-K partials
      return (M > 0 && N > 0) ? round16((size_t)M * N * sizeof(float)) +
                                    (M <= GEMV_MAX_M ? 16 : linear_ws_bytes(M, N, K))
                              : 0;
    case NVFP4_OP_GROUPED_SWIGLU:
      return (N > 0 && G > 0)
                 ? (size_t)grouped_swiglu_parts_bound(M > 0 ? M : 0, N, G) * sizeof(uint32_t)
                 : 0;
    case NVFP4_OP_GROUPED_RUN: return (M > 0 && K > 0) ? grouped_run_ws_bytes_any(M, K) : 0;
    case NVFP4_OP_MOE_RUN: return moe_ws_bytes_any(M, N, K, G);
    default: return 0;
  }
}

NVFP4_API int nvfp4_amax_gsa(const void* x, int x_dtype, int64_t numel, float* gsa, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!dtype_ok(x_dtype)) return NVFP4_ERR_DTYPE;
  if (numel < 0) return NVFP4_ERR_SHAPE;
  if (gsa == nullptr || (numel > 0 && x == nullptr)) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(gsa, 4)) return NVFP4_ERR_ALIGN;
  const size_t need = amax_ws_bytes(numel);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return NVFP4_ERR_ALIGN;
  }
  return launched(launch_amax_gsa(x, x_dtype == NVFP4_DTYPE_BF16, numel, gsa, ws,
                                  (hipStream_t)stream));
}

NVFP4_API int nvfp4_quantize_from_buffer(const void* x, int x_dtype, int64_t M, int64_t K,
                                         const float* gsa, uint8_t* codes, uint8_t* scales,
                                         void* stream) {
  if (!dtype_ok(x_dtype)) return NVFP4_ERR_DTYPE;
  if (M < 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (M > 0 && (M * (K / 16) + 255) / 256 > I32_MAX) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (x == nullptr || gsa == nullptr || codes == nullptr || scales == nullptr)
    return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(gsa, 4)) return NVFP4_ERR_ALIGN;
  return launched(launch_quantize(x, x_dtype == NVFP4_DTYPE_BF16, M, K, gsa, codes, scales,
                                  (hipStream_t)stream));
}

NVFP4_API int nvfp4_amax_quantize(const void* x, int x_dtype, int64_t M, int64_t K, float* gsa,
                                  uint8_t* codes, uint8_t* scales, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!dtype_ok(x_dtype)) return NVFP4_ERR_DTYPE;
  if (M < 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (M > 0 && (M * (K / 16) + 255) / 256 > I32_MAX) return NVFP4_ERR_SHAPE;
  if (gsa == nullptr) return NVFP4_ERR_NULL;
  if (!aligned(gsa, 4)) return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (M == 0)  // the amax of nothing: the 1e-8 floor
    return launched(launch_amax_finalize(nullptr, 0, gsa, s));
  if (x == nullptr || codes == nullptr || scales == nullptr) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 8)) return NVFP4_ERR_ALIGN;
  const bool bf16 = x_dtype == NVFP4_DTYPE_BF16;
  if (amax_quantize_small_ok(M, K))  // one workgroup: amax, gsa and codes in one kernel
    return launched(launch_amax_quantize_small(x, bf16, M, K, gsa, codes, scales, s));
  const size_t need = amax_ws_bytes(M * K);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return NVFP4_ERR_ALIGN;
  }
  return launched(launch_amax_then_quantize(x, bf16, M, K, gsa, codes, scales, ws, s));
}

NVFP4_API int nvfp4_rmsnorm_quantize(const void* x, int x_dtype, const void* norm_weight,
                                     int w_dtype, float eps, int64_t M, int64_t K,
                                     int gsa_per_row, float* gsa, float* inv_rms,
                                     uint8_t* codes, uint8_t* scales, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype)) return NVFP4_ERR_DTYPE;
  if (M < 0 || K <= 0 || K % 16 != 0 || M > I32_MAX) return NVFP4_ERR_SHAPE;
  if (!(eps > 0.0f) || eps > 3.0e38f) return NVFP4_ERR_SHAPE;  // a zero row stays finite
  if (M > 0 && (M * (K / 8) + 255) / 256 > I32_MAX) return NVFP4_ERR_SHAPE;
  if (gsa == nullptr) return NVFP4_ERR_NULL;
  if (!aligned(gsa, 4)) return NVFP4_ERR_ALIGN;
  const bool per_row = gsa_per_row != 0;
  if (M == 0)  // one scale of nothing: the 1e-8 floor; per-row: nothing to write
    return per_row ? NVFP4_OK
                   : launched(launch_amax_finalize(nullptr, 0, gsa, (hipStream_t)stream));
  if (!x || !norm_weight || !inv_rms || !codes || !scales) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(norm_weight, 16) || !aligned(codes, 8) ||
      !aligned(inv_rms, 4))
    return NVFP4_ERR_ALIGN;
  if (!per_row) {
    if (ws == nullptr || ws_bytes < (size_t)M * sizeof(uint32_t)) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return NVFP4_ERR_ALIGN;
  }
  return launched(launch_rmsnorm_quantize(x, x_dtype == NVFP4_DTYPE_BF16, norm_weight,
                                          w_dtype == NVFP4_DTYPE_BF16, eps, M, K, per_row, gsa,
                                          inv_rms, codes, scales, (uint32_t*)ws,
                                          (hipStream_t)stream));
}

NVFP4_API int nvfp4_quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, float* ws2,
                                    uint8_t* codes, uint8_t* scales, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!dtype_ok(w_dtype)) return NVFP4_ERR_DTYPE;
  if (N <= 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if ((N * (K / 16) + 255) / 256 > I32_MAX) return NVFP4_ERR_SHAPE;
  if (w == nullptr || ws2 == nullptr || codes == nullptr || scales == nullptr)
    return NVFP4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(codes, 8) || !aligned(ws2, 4)) return NVFP4_ERR_ALIGN;
  const size_t need = amax_ws_bytes(N * K);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return NVFP4_ERR_ALIGN;
  }
  const bool bf16 = w_dtype == NVFP4_DTYPE_BF16;
  const hipError_t e = launch_amax_gsa(w, bf16, N * K, ws2, ws, (hipStream_t)stream);
  if (e != hipSuccess) return launched(e);
  return launched(launch_quantize(w, bf16, N, K, ws2, codes, scales, (hipStream_t)stream));
}

static int linear_impl(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2, void* y,
                       int y_dtype, int64_t M, int64_t N, int64_t K, bool gsa_rows, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  int st = check_gemm_shape(M, N, K);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !gsa || !w_codes || !w_scales || !ws2 || !y) return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 8) || !aligned(w_codes, 8) || !aligned(gsa, 4) || !aligned(ws2, 4) ||
      !aligned(y, y_dtype == NVFP4_DTYPE_FP32 ? 4 : 2))
    return NVFP4_ERR_ALIGN;
  const bool ybf = y_dtype == NVFP4_DTYPE_BF16;
  hipStream_t s = (hipStream_t)stream;
  if (M <= GEMV_MAX_M)
    return launched(
        launch_gemv(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, ybf, M, N, K, s, gsa_rows));
  return launched(launch_gemm(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, ybf, M, N, K, s,
                              gsa_rows, ws, ws_bytes));
}

NVFP4_API int nvfp4_linear(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                           const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                           void* y, int y_dtype, int64_t M, int64_t N, int64_t K, void* ws,
                           size_t ws_bytes, void* stream) {
  return linear_impl(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_dtype, M, N, K, false,
                     ws, ws_bytes, stream);
}

NVFP4_API int nvfp4_linear_rows(const uint8_t* a_codes, const uint8_t* a_scales,
                                const float* gsa_rows, const uint8_t* w_codes,
                                const uint8_t* w_scales, const float* ws2, void* y, int y_dtype,
                                int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                                void* stream) {
  return linear_impl(a_codes, a_scales, gsa_rows, w_codes, w_scales, ws2, y, y_dtype, M, N, K,
                     true, ws, ws_bytes, stream);
}

NVFP4_API int nvfp4_router_topk(const uint8_t* a_codes, const uint8_t* a_scales,
                                const float* gsa, const uint8_t* w_codes, const uint8_t* w_scales,
                                const float* ws2, const float* bias, int64_t M, int64_t N,
                                int64_t K, int topk, int32_t* topk_idx, float* topk_score,
                                void* ws, size_t ws_bytes, void* stream) {
  int st = check_gemm_shape(M, N, K);
  if (st != NVFP4_OK) return st;
  if (N < 1 || N > ROUTER_MAX_N || topk < 1 || topk > N || topk > ROUTER_MAX_K)
    return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !gsa || !w_codes || !w_scales || !ws2 || !topk_idx ||
      !topk_score)
    return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 8) || !aligned(w_codes, 8) || !aligned(gsa, 4) || !aligned(ws2, 4) ||
      !aligned(topk_idx, 4) || !aligned(topk_score, 4) || (bias && !aligned(bias, 4)))
    return NVFP4_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < (size_t)M * N * sizeof(float)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  float* logits = (float*)ws;
  const size_t lbytes = round16((size_t)M * N * sizeof(float));
  hipStream_t s = (hipStream_t)stream;
  if (M <= GEMV_MAX_M) {
    // one launch: the gate linear's last workgroup chooses the experts; its
    // ticket counter is the word after the logits
    if (ws_bytes < lbytes + 16) return NVFP4_ERR_WORKSPACE;
    RouterEpilogue r{topk, bias, topk_idx, topk_score, (uint32_t*)((uint8_t*)ws + lbytes)};
    return launched(launch_gemv(a_codes, a_scales, gsa, w_codes, w_scales, ws2, logits, false, M,
                                N, K, s, false, &r));
  }
  // the bytes after the logits, if any, take the linear's split-K partials
  void* lws = ws_bytes > lbytes ? (void*)((uint8_t*)ws + lbytes) : nullptr;
  const size_t lws_bytes = ws_bytes > lbytes ? ws_bytes - lbytes : 0;
  // a split-K gate linear leaves its partials after the logits: the choice
  // kernel adds and scales them (and writes the logits) itself
  int nsplit = 0;
  const hipError_t e = launch_gemm(a_codes, a_scales, gsa, w_codes, w_scales, ws2, logits, false,
                                   M, N, K, s, false, lws, lws_bytes, &nsplit);
  if (e != hipSuccess) return launched(e);
  return launched(launch_router_topk(nsplit ? (const float*)lws : logits, nsplit, gsa, ws2,
                                     logits, bias, M, N, topk, topk_idx, topk_score, s));
}

// One-row decodes from this many weight rows on take the ring (measured on
// an MI355X at K = 7168: 16384 rows 22.5 us either way, 32768 rows 27.5 us
// against 42.7 us with 8 rows a workgroup).
constexpr int64_t RUN_RING_MIN_N = 24576;
// Activations of at most this many elements are reduced by every workgroup
// of a grouped run itself (one launch); larger ones take a phase-1 launch.
constexpr int64_t GROUPED_RUN_X_NUMEL = 16384;

namespace nvfp4 {
// The argument checks of nvfp4_linear_run that come before any launch (the
// workspace is checked where a path needs it).
int linear_run_check(const void* x, int x_dtype, const float* gsa, const uint8_t* codes,
                     const uint8_t* scales, const uint8_t* w_codes, const uint8_t* w_scales,
                     const float* ws2, const void* y, int y_dtype, int64_t M, int64_t N,
                     int64_t K) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  int st = check_gemm_shape(M, N, K);
  if (st != NVFP4_OK) return st;
  if (M > 0 && (M * (K / 16) + 255) / 256 > I32_MAX) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!x || !gsa || !codes || !scales || !w_codes || !w_scales || !ws2 || (N > 0 && !y))
    return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(gsa, 4) || !aligned(w_codes, 8) ||
      !aligned(ws2, 4) || !aligned(y, y_dtype == NVFP4_DTYPE_FP32 ? 4 : 2))
    return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}
}  // namespace nvfp4

NVFP4_API int nvfp4_linear_run(const void* x, int x_dtype, float* gsa, uint8_t* codes,
                               uint8_t* scales, const uint8_t* w_codes, const uint8_t* w_scales,
                               const float* ws2, void* y, int y_dtype, int64_t M, int64_t N,
                               int64_t K, void* ws, size_t ws_bytes, void* stream) {
  const int st = linear_run_check(x, x_dtype, gsa, codes, scales, w_codes, w_scales, ws2, y,
                                  y_dtype, M, N, K);
  if (st != NVFP4_OK || M == 0) return st;
  const bool xbf = x_dtype == NVFP4_DTYPE_BF16, ybf = y_dtype == NVFP4_DTYPE_BF16;
  hipStream_t s = (hipStream_t)stream;
  // decode shapes with a long weight stream (N >= RUN_RING_MIN_N): one
  // kernel, the weight-streaming ring with 128 rows per workgroup, each
  // workgroup quantizing the activation itself
  if (N >= RUN_RING_MIN_N && M * K <= GROUPED_RUN_X_NUMEL && M <= 2 &&
      grouped_run_supported(M, K, x, w_codes, w_scales))
    return launched(launch_grouped_run(x, xbf, M, nullptr, 0, gsa, codes, scales, nullptr,
                                       nullptr, 1, M, w_codes, w_scales, ws2, y, ybf, N, K, false,
                                       0, 0.f, nullptr, nullptr, s));
  // other decode shapes: one kernel, 8 weight rows per workgroup (4 when N
  // is small), every workgroup quantizes the activation itself
  const bool one_kernel = N > 0 && !linear_run_prefers_two_launches(M, N);
  if (one_kernel && gemv_narrow_run_supported(M, K, x, w_codes, w_scales))
    return launched(launch_narrow_run(x, xbf, gsa, codes, scales, w_codes, w_scales, ws2, y, ybf,
                                      M, N, K, s));
  if (one_kernel && gemv_run_supported(M, K, x, w_codes, w_scales))
    return launched(launch_gemv_run(x, xbf, gsa, codes, scales, w_codes, w_scales, ws2, y, ybf, M,
                                    N, K, s));
  // general case: steps 1-2 (one kernel for a small activation), then step 3
  hipError_t e = hipSuccess;
  if (amax_quantize_small_ok(M, K)) {
    e = launch_amax_quantize_small(x, xbf, M, K, gsa, codes, scales, s);
  } else {
    const size_t need = amax_ws_bytes(M * K);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 4)) return NVFP4_ERR_ALIGN;
    e = launch_amax_then_quantize(x, xbf, M, K, gsa, codes, scales, ws, s);
  }
  if (e == hipSuccess && N > 0) {
    if (M <= GEMV_MAX_M)
      e = launch_gemv(codes, scales, gsa, w_codes, w_scales, ws2, y, ybf, M, N, K, s);
    else  // the amax partials are consumed by now: the workspace takes the split K
      e = launch_gemm(codes, scales, gsa, w_codes, w_scales, ws2, y, ybf, M, N, K, s, false, ws,
                      ws_bytes);
  }
  return launched(e);
}

NVFP4_API int nvfp4_grouped_linear(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const float* gsa, int64_t a_rows, const int32_t* row_index,
                                   const int32_t* group_offsets, int G, int64_t M_total,
                                   const uint8_t* w_codes, const uint8_t* w_scales,
                                   const float* ws2, void* y, int y_dtype, int64_t N, int64_t K,
                                   void* stream) {
  if (!dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  int st = check_gemm_shape(M_total, N, K);
  if (st != NVFP4_OK) return st;
  if (G < 1 || G > 65535 || a_rows < 0 || a_rows > I32_MAX) return NVFP4_ERR_SHAPE;
  if (row_index == nullptr && a_rows < M_total) return NVFP4_ERR_SHAPE;
  if (M_total == 0 || N == 0) return NVFP4_OK;
  if (a_rows == 0) return NVFP4_ERR_SHAPE;
  if (!a_codes || !a_scales || !gsa || !group_offsets || !w_codes || !w_scales || !ws2 || !y)
    return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 8) || !aligned(w_codes, 8) || !aligned(gsa, 4) || !aligned(ws2, 4) ||
      !aligned(group_offsets, 4) || !aligned(row_index, 4) ||
      !aligned(y, y_dtype == NVFP4_DTYPE_FP32 ? 4 : 2))
    return NVFP4_ERR_ALIGN;
  return launched(launch_grouped_gemv(a_codes, a_scales, gsa, a_rows, row_index, group_offsets, G,
                                      M_total, w_codes, w_scales, ws2, y,
                                      y_dtype == NVFP4_DTYPE_BF16, N, K, (hipStream_t)stream));
}

NVFP4_API int nvfp4_grouped_linear_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                          const float* gsa, int64_t a_rows,
                                          const int32_t* row_index, const int32_t* group_offsets,
                                          int G, int64_t M_total, const uint8_t* w_codes,
                                          const uint8_t* w_scales, const float* ws2, float* h,
                                          float* gsa_h, uint8_t* h_codes, uint8_t* h_scales,
                                          int64_t N_inter, int64_t K, int granularity,
                                          float limit, void* ws, size_t ws_bytes, void* stream) {
  int st = check_gemm_shape(M_total, N_inter, K);
  if (st != NVFP4_OK) return st;
  if (limit != limit) return NVFP4_ERR_SHAPE;  // NaN limit
  if (G < 1 || G > 65535 || a_rows < 0 || a_rows > I32_MAX) return NVFP4_ERR_SHAPE;
  if (row_index == nullptr && a_rows < M_total) return NVFP4_ERR_SHAPE;
  if (granularity < 1 || N_inter % (2 * (int64_t)granularity) != 0) return NVFP4_ERR_SHAPE;
  if (gsa_h == nullptr) return NVFP4_ERR_NULL;
  if (!aligned(gsa_h, 4)) return NVFP4_ERR_ALIGN;
  if ((h_codes == nullptr) != (h_scales == nullptr)) return NVFP4_ERR_NULL;  // both or neither
  if (h_codes != nullptr && (N_inter / 2) % 16 != 0) return NVFP4_ERR_SHAPE;
  if (h_codes != nullptr && !aligned(h_codes, 8)) return NVFP4_ERR_ALIGN;
  // h's quantize reads h in 16-byte vectors
  if (h_codes != nullptr && h != nullptr && !aligned(h, 16)) return NVFP4_ERR_ALIGN;
  if (M_total == 0 || N_inter == 0)  // the amax of nothing: gsa_h from the 1e-8 floor
    return launched(launch_amax_finalize(nullptr, 0, gsa_h, (hipStream_t)stream));
  if (a_rows == 0) return NVFP4_ERR_SHAPE;
  if (!a_codes || !a_scales || !gsa || !group_offsets || !w_codes || !w_scales || !ws2 || !h)
    return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(a_scales, 16) || !aligned(w_codes, 16) ||
      !aligned(w_scales, 16) || !aligned(gsa, 4) || !aligned(ws2, 4) ||
      !aligned(group_offsets, 4) || !aligned(row_index, 4) || !aligned(h, 4))
    return NVFP4_ERR_ALIGN;
  if (!grouped_swiglu_supported(N_inter, K, granularity, a_rows, a_codes, a_scales, w_codes,
                                w_scales))
    return NVFP4_ERR_SHAPE;
  const size_t need = (size_t)grouped_swiglu_parts_for(a_codes, a_scales, w_codes, w_scales,
                                                       a_rows, M_total, G, N_inter, K) *
                      sizeof(uint32_t);
  if (ws == nullptr || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return NVFP4_ERR_ALIGN;
  return launched(launch_grouped_swiglu(a_codes, a_scales, gsa, a_rows, row_index, group_offsets,
                                        G, M_total, w_codes, w_scales, ws2, h, gsa_h, N_inter, K,
                                        granularity, limit, (uint32_t*)ws, h_codes, h_scales,
                                        (hipStream_t)stream));
}

NVFP4_API int nvfp4_swiglu_deinterleave(const float* l1, float* h, int64_t M, int64_t N_inter,
                                        int granularity, float limit, void* stream) {
  if (M < 0 || granularity < 1 || N_inter < 0 || N_inter % (2 * (int64_t)granularity) != 0)
    return NVFP4_ERR_SHAPE;
  if (limit != limit) return NVFP4_ERR_SHAPE;  // NaN limit
  if ((M * (N_inter / 2) + 255) / 256 > I32_MAX) return NVFP4_ERR_SHAPE;
  if (M == 0 || N_inter == 0) return NVFP4_OK;
  if (l1 == nullptr || h == nullptr) return NVFP4_ERR_NULL;
  if (!aligned(l1, 4) || !aligned(h, 4)) return NVFP4_ERR_ALIGN;
  return launched(
      launch_swiglu_deinterleave(l1, h, M, N_inter, granularity, limit, (hipStream_t)stream));
}

// ---------------------------------------------------------------- runs
// At most this many amax partials are reduced by every workgroup of the
// second expert projection itself.
constexpr int64_t RUN_INLINE_PARTS = 2048;

static size_t grouped_run_ws_bytes(int64_t rows, int64_t K) {
  return rows * K > GROUPED_RUN_X_NUMEL ? (size_t)amax_parts_for(rows * K) * sizeof(uint32_t) : 0;
}

static int check_grouped(int64_t a_rows, const int32_t* row_index, int G, int64_t M_total,
                         int64_t N, int64_t K) {
  int st = check_gemm_shape(M_total, N, K);
  if (st != NVFP4_OK) return st;
  if (G < 1 || G > 65535 || a_rows < 0 || a_rows > I32_MAX) return NVFP4_ERR_SHAPE;
  if (row_index == nullptr && a_rows < M_total) return NVFP4_ERR_SHAPE;
  if (a_rows > 0 && (a_rows * (K / 16) + 255) / 256 > I32_MAX) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

NVFP4_API int nvfp4_grouped_linear_run(const void* x, int x_dtype, int64_t x_rows, float* gsa,
                                       uint8_t* x_codes, uint8_t* x_scales,
                                       const int32_t* row_index, const int32_t* group_offsets,
                                       int G, int64_t M_total, const uint8_t* w_codes,
                                       const uint8_t* w_scales, const float* ws2, void* y,
                                       int y_dtype, int64_t N, int64_t K, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  int st = check_grouped(x_rows, row_index, G, M_total, N, K);
  if (st != NVFP4_OK) return st;
  if (gsa == nullptr) return NVFP4_ERR_NULL;
  if (!aligned(gsa, 4)) return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (x_rows == 0)  // the amax of nothing: the 1e-8 floor; no row to read
    return M_total == 0 || N == 0 ? launched(launch_amax_finalize(nullptr, 0, gsa, s))
                                  : NVFP4_ERR_SHAPE;
  if (!x || !x_codes || !x_scales || !group_offsets || !w_codes || !w_scales || !ws2 ||
      (M_total > 0 && N > 0 && !y))
    return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x_codes, 8) || !aligned(w_codes, 8) || !aligned(ws2, 4) ||
      !aligned(group_offsets, 4) || !aligned(row_index, 4) ||
      !aligned(y, y_dtype == NVFP4_DTYPE_FP32 ? 4 : 2))
    return NVFP4_ERR_ALIGN;
  const bool xbf = x_dtype == NVFP4_DTYPE_BF16, ybf = y_dtype == NVFP4_DTYPE_BF16;
  const int64_t numel = x_rows * K;
  if (M_total > 0 && N > 0 && grouped_run_supported(x_rows, K, x, w_codes, w_scales)) {
    if (numel <= GROUPED_RUN_X_NUMEL)  // one launch: every workgroup takes the amax of x
      return launched(launch_grouped_run(x, xbf, x_rows, nullptr, 0, gsa, x_codes, x_scales,
                                         row_index, group_offsets, G, M_total, w_codes, w_scales,
                                         ws2, y, ybf, N, K, false, 0, 0.f, nullptr, nullptr, s));
    // two launches: the amax partials, then the grouped linear, every
    // workgroup of which reduces them -- unless the groups are large enough
    // for the tiled kernel, which reads codes quantized beforehand
    if ((M_total + G - 1) / G < GROUPED_MFMA_MIN_ROWS) {
      const size_t need = grouped_run_ws_bytes(x_rows, K);
      if (ws == nullptr || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
      if (!aligned(ws, 4)) return NVFP4_ERR_ALIGN;
      int64_t np = 0;
      hipError_t e = launch_amax_partials(x, xbf, numel, (uint32_t*)ws, &np, s);
      if (e != hipSuccess) return launched(e);
      return launched(launch_grouped_run(x, xbf, x_rows, (const uint32_t*)ws, np, gsa, x_codes,
                                         x_scales, row_index, group_offsets, G, M_total, w_codes,
                                         w_scales, ws2, y, ybf, N, K, false, 0, 0.f, nullptr,
                                         nullptr, s));
    }
  }
  // otherwise steps 1-2 as nvfp4_amax_quantize, then nvfp4_grouped_linear
  hipError_t e;
  if (amax_quantize_small_ok(x_rows, K)) {
    e = launch_amax_quantize_small(x, xbf, x_rows, K, gsa, x_codes, x_scales, s);
  } else {
    const size_t need = amax_ws_bytes(numel);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 4)) return NVFP4_ERR_ALIGN;
    e = launch_amax_then_quantize(x, xbf, x_rows, K, gsa, x_codes, x_scales, ws, s);
  }
  if (e != hipSuccess || M_total == 0 || N == 0) return launched(e);
  return launched(launch_grouped_gemv(x_codes, x_scales, gsa, x_rows, row_index, group_offsets, G,
                                      M_total, w_codes, w_scales, ws2, y, ybf, N, K, s));
}

// The amax partials of x, or of h after the first projection: the
// weight-streaming kernel's, or the tiled kernel's for up to T * E pairs
// (every token at most once per expert); a call checks its own pair count.
static size_t moe_ws_bytes(int64_t T, int64_t N1, int64_t K1, int E) {
  const size_t a = T > 0 ? amax_ws_bytes(T * K1) : 0;
  const size_t b = (N1 > 0 && E > 0 && T > 0)
                       ? (size_t)grouped_swiglu_parts_bound(T * E, N1, E) * sizeof(uint32_t)
                       : 0;
  return a > b ? a : b;
}

NVFP4_API int nvfp4_moe_run(const void* x, int x_dtype, int64_t T, float* gsa_x,
                            uint8_t* x_codes, uint8_t* x_scales, const int32_t* row_index,
                            const int32_t* group_offsets, int E, int64_t P,
                            const uint8_t* w1_codes, const uint8_t* w1_scales,
                            const float* w1_ws2, int64_t N1, int64_t K1, int granularity,
                            float limit, float* h, float* gsa_h, uint8_t* h_codes,
                            uint8_t* h_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                            const float* w2_ws2, int64_t N2, void* y, int y_dtype, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return NVFP4_ERR_DTYPE;
  if (limit != limit) return NVFP4_ERR_SHAPE;  // NaN limit
  if (T < 1 || P < 0 || N1 <= 0 || N2 <= 0) return NVFP4_ERR_SHAPE;
  if (row_index == nullptr) return NVFP4_ERR_NULL;
  int st = check_grouped(T, row_index, E, P, N1, K1);
  if (st != NVFP4_OK) return st;
  const int64_t K2 = N1 / 2;
  if (K2 % 256 != 0) return NVFP4_ERR_SHAPE;
  if (check_gemm_shape(P, N2, K2) != NVFP4_OK) return NVFP4_ERR_SHAPE;
  if (!x || !gsa_x || !x_codes || !x_scales || !group_offsets || !w1_codes || !w1_scales ||
      !w1_ws2 || !h || !gsa_h || !h_codes || !h_scales || !w2_codes || !w2_scales || !w2_ws2 ||
      !y || !ws)
    return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x_codes, 16) || !aligned(x_scales, 16) ||
      !aligned(w1_codes, 16) || !aligned(w1_scales, 16) || !aligned(w2_codes, 16) ||
      !aligned(w2_scales, 16) || !aligned(h, 16) || !aligned(h_codes, 16) ||
      !aligned(h_scales, 16) || !aligned(gsa_x, 4) || !aligned(gsa_h, 4) ||
      !aligned(w1_ws2, 4) || !aligned(w2_ws2, 4) || !aligned(group_offsets, 4) ||
      !aligned(row_index, 4) || !aligned(ws, 4) ||
      !aligned(y, y_dtype == NVFP4_DTYPE_FP32 ? 4 : 2))
    return NVFP4_ERR_ALIGN;
  if (!grouped_swiglu_supported(N1, K1, granularity, T, x_codes, x_scales, w1_codes, w1_scales) ||
      !grouped_run_supported(T, K1, x, w1_codes, w1_scales) ||
      !grouped_run_supported(P > 0 ? P : 1, K2, h, w2_codes, w2_scales))
    return NVFP4_ERR_SHAPE;
  if (ws_bytes < moe_ws_bytes(T, N1, K1, E) ||
      ws_bytes < (size_t)grouped_swiglu_parts_for(x_codes, x_scales, w1_codes, w1_scales, T, P, E,
                                                  N1, K1) *
                     sizeof(uint32_t))
    return NVFP4_ERR_WORKSPACE;
  const bool xbf = x_dtype == NVFP4_DTYPE_BF16, ybf = y_dtype == NVFP4_DTYPE_BF16;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* parts = (uint32_t*)ws;
  if (P == 0) {  // no pair: x is still quantized; h's amax is of nothing
    hipError_t e = amax_quantize_small_ok(T, K1)
                       ? launch_amax_quantize_small(x, xbf, T, K1, gsa_x, x_codes, x_scales, s)
                       : launch_amax_then_quantize(x, xbf, T, K1, gsa_x, x_codes, x_scales, ws, s);
    if (e != hipSuccess) return launched(e);
    return launched(launch_amax_finalize(nullptr, 0, gsa_h, s));
  }
  // first projection with SwiGLU: its workgroups quantize x themselves when
  // x is small, else x is quantized first
  int64_t np = 0;
  hipError_t e;
  if (T * K1 <= GROUPED_RUN_X_NUMEL) {
    e = launch_grouped_run(x, xbf, T, nullptr, 0, gsa_x, x_codes, x_scales, row_index,
                           group_offsets, E, P, w1_codes, w1_scales, w1_ws2, h, false, N1, K1,
                           true, granularity, limit, parts, &np, s);
  } else {
    e = amax_quantize_small_ok(T, K1)
            ? launch_amax_quantize_small(x, xbf, T, K1, gsa_x, x_codes, x_scales, s)
            : launch_amax_then_quantize(x, xbf, T, K1, gsa_x, x_codes, x_scales, ws, s);
    if (e == hipSuccess)
      e = launch_grouped_swiglu_l1(x_codes, x_scales, gsa_x, T, row_index, group_offsets, E, P,
                                   w1_codes, w1_scales, w1_ws2, h, N1, K1, granularity, limit,
                                   parts, &np, s);
  }
  if (e != hipSuccess) return launched(e);
  // second projection: with few partials its workgroups reduce them and
  // quantize their rows of h themselves; else, or when the groups are large
  // enough for the tiled kernel, h is quantized first
  if (np <= RUN_INLINE_PARTS && (P + E - 1) / E < GROUPED_MFMA_MIN_ROWS)
    return launched(launch_grouped_run(h, false, P, parts, np, gsa_h, h_codes, h_scales, nullptr,
                                       group_offsets, E, P, w2_codes, w2_scales, w2_ws2, y, ybf,
                                       N2, K2, false, 0, 0.f, nullptr, nullptr, s));
  e = launch_amax_finalize(parts, np, gsa_h, s);
  if (e == hipSuccess) e = launch_quantize(h, false, P, K2, gsa_h, h_codes, h_scales, s);
  if (e == hipSuccess)
    e = launch_grouped_gemv(h_codes, h_scales, gsa_h, P, nullptr, group_offsets, E, P, w2_codes,
                            w2_scales, w2_ws2, y, ybf, N2, K2, s);
  return launched(e);
}

static size_t grouped_run_ws_bytes_any(int64_t rows, int64_t K) {
  const size_t a = grouped_run_ws_bytes(rows, K), b = amax_ws_bytes(rows * K);
  return a > b ? a : b;
}

static size_t moe_ws_bytes_any(int64_t T, int64_t N1, int64_t K1, int E) {
  return moe_ws_bytes(T, N1, K1, E);
}
