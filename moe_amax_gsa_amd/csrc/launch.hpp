// launch.hpp -- internal launchers behind the C ABI (not exported).
// Each launcher assumes its arguments were validated by the ABI layer and
// returns the HIP status of its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Allow `bytes` of dynamic LDS for kernel f on the current device.  The
// attribute belongs to the device, so it is set once per device; `done` is
// the calling launcher's record for that kernel (setting it twice from two
// threads is harmless).
inline hipError_t allow_dynamic_lds(const void* f, int bytes, unsigned char (&done)[64]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool track = dev >= 0 && dev < 64;
  if (track && done[dev]) return hipSuccess;
  e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && track) done[dev] = 1;
  return e;
}

// amax -> gsa
constexpr int64_t AMAX_SMALL_NUMEL = 65536;  // one workgroup, one kernel
constexpr int AMAX_MAX_PARTS = 1024;         // phase-1 workgroups at most
int amax_parts_for(int64_t numel);
hipError_t launch_amax_gsa(const void* x, bool bf16, int64_t numel, float* gsa, void* ws,
                           hipStream_t s);

// Phase 1 alone: amax_parts_for(numel) partial maxima (bits in x's format)
// into partials; their count in *nparts.
hipError_t launch_amax_partials(const void* x, bool bf16, int64_t numel, uint32_t* partials,
                                int64_t* nparts, hipStream_t s);

// amax -> gsa -> quantize in one workgroup (at most 4096 blocks)
bool amax_quantize_small_ok(int64_t M, int64_t K);
hipError_t launch_amax_quantize_small(const void* x, bool bf16, int64_t M, int64_t K, float* gsa,
                                      uint8_t* codes, uint8_t* scales, hipStream_t s);

// steps 1-2 past the one-workgroup size: two-phase amax, then the quantize
// (which reduces few partials itself); ws holds amax_parts_for(M K) partials
hipError_t launch_amax_then_quantize(const void* x, bool bf16, int64_t M, int64_t K, float* gsa,
                                     uint8_t* codes, uint8_t* scales, void* ws, hipStream_t s);

// quantize from a device gsa
hipError_t launch_quantize(const void* x, bool bf16, int64_t M, int64_t K, const float* gsa,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);

// SwiGLU de-interleave (limit > 0: gate capped at limit, up clamped to +-limit)
hipError_t launch_swiglu_deinterleave(const float* l1, float* h, int64_t M, int64_t NI, int gran,
                                      float limit, hipStream_t s);

// RMSNorm + quantize: per-row gsa (M,) or one gsa (then `partials` holds M
// row maxima).
hipError_t launch_rmsnorm_quantize(const void* x, bool x_bf16, const void* w, bool w_bf16,
                                   float eps, int64_t M, int64_t K, bool per_row, float* gsa,
                                   float* inv_rms, uint8_t* codes, uint8_t* scales,
                                   uint32_t* partials, hipStream_t s);

// Router expert choice on fp32 logits (M, N), N <= ROUTER_MAX_N,
// 1 <= k <= min(N, ROUTER_MAX_K):
// idx (M, k) and score (M, k) = sqrt(softplus(logit)) of the chosen experts.
constexpr int64_t ROUTER_MAX_N = 1024;
constexpr int ROUTER_MAX_K = 64;
// The logits are src (nsrc == 0), or the sum of nsrc split-K partials
// (split z at src + z * M * N) times gsa[0] * ws2[0], then also written to
// logits.
hipError_t launch_router_topk(const float* src, int nsrc, const float* gsa, const float* ws2,
                              float* logits, const float* bias, int64_t M, int64_t N, int k,
                              int32_t* idx, float* score, hipStream_t s);

// Phase 2 of an amax over partials, then the quantize of fp32 x (M, K):
// below 2^20 half-blocks fused (every quantize workgroup reduces the
// partials itself, workgroup 0 writes gsa), from there a finalize launch
// and the quantize.
hipError_t launch_quantize_finalize(const float* x, int64_t M, int64_t K,
                                    const uint32_t* partials, int64_t nparts, float* gsa,
                                    uint8_t* codes, uint8_t* scales, hipStream_t s);

// Phase 2 of an amax over partials (bits of non-negative fp32 maxima): gsa.
hipError_t launch_amax_finalize(const uint32_t* partials, int64_t nparts, float* gsa,
                                hipStream_t s);

// Weight-streaming linear for few rows (FP4 matrix cores).
constexpr int64_t GEMV_MAX_M = 16;
// Up to GEMV_MAX_M rows against many weight rows.  Measured on MI355X with
// cold weights, K = 7168: one or two rows from 8192 weight rows, and three
// or four from 10240, stream faster through the weight ring (one group) than
// through the few-row kernels (4 x 16384: 24.1 against 47.4 us; 1 x 12288:
// 13.2 against 16.7 us; 2 x 8192: 11.2 against 13.2 us; at 4096 rows the
// few-row kernels win, 6.2 against 10.6 us).  The tiled GEMM (unsplit: its
// time hardly moves from 5 to 16 rows) is faster from 8 rows and 10240
// weight rows (12 x 10240: 29.4 against 36.7 us; 16 x 16384: 32.8 against
// 57.4 us; 8 x 8192: 23.4 against 21.6 on the rows kernel, so not there),
// from 15 rows and 6144 weight rows (16 x 6144: 27.4 against 29.2 us; 12 x
// 8192: 28.7 against 25.8, so not there) and from 5 rows and 16384 weight
// rows (5 x 16384: 32.4 against 37.3 us; 5 x 12288: 30 against 28.6, so not
// there).
// Three or four rows take the 16-row kernel from 3072 weight rows up to the
// ring's range, which for them starts at 10240 (4 x 3072: 9.3 against 13.1
// us on the 4-row kernel; 4 x 8192: 17.0 against 25.3, and 22.3 on the ring;
// 4 x 1536: 8.9 against 7.4, so not there; 4 x 10240: 23.6 against 22.8 on
// the ring).
inline bool gemv_ring_preferred(int64_t M, int64_t N) {
  return (M <= 2 && N >= 8192) || (M <= 4 && N >= 10240);
}
inline bool gemv_narrow_preferred(int64_t M, int64_t N) { return M <= 2 || N < 3072; }
inline bool gemv_tiled_preferred(int64_t M, int64_t N) {
  return (M >= 15 && N >= 6144) || (M >= 8 && N >= 10240) || (M >= 5 && N >= 16384);
}
// The linear run of so few rows: its one-kernel forms (every workgroup
// quantizes the activation itself) lose to a quantize launch followed by the
// ring or the tiles above, except for one row against under 12288 weight rows
// (2 x 12288: 16.9 against 28.7 us; 2 x 8192: 15.4 against 20.5 us;
// 1 x 8192: 15.7 against 13.4 us).
inline bool linear_run_prefers_two_launches(int64_t M, int64_t N) {
  return (gemv_ring_preferred(M, N) && (M > 1 || N >= 12288)) || gemv_tiled_preferred(M, N);
}
// The dense router's choice run by the linear's last workgroup: k experts
// per row of the fp32 logits the linear writes to y (M, N <= 1024), bias
// (N,) or NULL, outputs idx / score (M, k), and a ticket counter that is
// zero before the launch and left zero after it.
struct RouterEpilogue {
  int k;
  const float* bias;
  int32_t* idx;
  float* score;
  uint32_t* count;
};
// gsa_rows: gsa holds one global scale per row (gsa[m]).  router: the choice
// in the same launch (y fp32).
hipError_t launch_gemv(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                       void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s,
                       bool gsa_rows = false, const RouterEpilogue* router = nullptr);

// Grouped weight-streaming linear (device-side group sizes).
hipError_t launch_grouped_gemv(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                               int64_t a_rows, const int32_t* row_index, const int32_t* offsets,
                               int G, int64_t M_total, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* ws2, void* y, bool y_bf16,
                               int64_t N, int64_t K, hipStream_t s);

// Grouped linear with SwiGLU, de-interleave and the first amax phase of h
// in its epilogue, then the second phase (gsa_h).  ws holds
// grouped_swiglu_parts_for(...) partials: grouped_swiglu_parts(N, G) for the
// weight-streaming kernel, grouped_tile_blocks(M_total, G, N) when the
// groups are large enough for the tiled one; grouped_swiglu_parts_bound is
// the larger of the two where the tiled one may run.  false: the operands
// or shape do not suit the fused kernels (nothing launched).
bool grouped_swiglu_supported(int64_t N, int64_t K, int gran, int64_t a_rows,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const uint8_t* w_codes, const uint8_t* w_scales);
int64_t grouped_swiglu_parts(int64_t N, int G);
int64_t grouped_swiglu_parts_for(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const uint8_t* w_codes, const uint8_t* w_scales, int64_t a_rows,
                                 int64_t M_total, int G, int64_t N, int64_t K);
int64_t grouped_swiglu_parts_bound(int64_t M_total, int64_t N, int G);
hipError_t launch_grouped_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* gsa, int64_t a_rows, const int32_t* row_index,
                                 const int32_t* offsets, int G, int64_t M_total,
                                 const uint8_t* w_codes, const uint8_t* w_scales,
                                 const float* ws2, float* h, float* gsa_h, int64_t N, int64_t K,
                                 int gran, float limit, uint32_t* partials, uint8_t* h_codes,
                                 uint8_t* h_scales, hipStream_t s);

// The gate/up linear with SwiGLU, de-interleave and the first amax phase of
// h (one partial per workgroup into partials, their count in *nparts), and
// nothing after it.
hipError_t launch_grouped_swiglu_l1(const uint8_t* a_codes, const uint8_t* a_scales,
                                    const float* gsa, int64_t a_rows, const int32_t* row_index,
                                    const int32_t* offsets, int G, int64_t M_total,
                                    const uint8_t* w_codes, const uint8_t* w_scales,
                                    const float* ws2, float* h, int64_t N, int64_t K, int gran,
                                    float limit, uint32_t* partials, int64_t* nparts,
                                    hipStream_t s);

// amax -> gsa -> quantize -> linear in one kernel for a few activation rows.
constexpr int64_t GEMV_RUN_MAX_M = 16;
constexpr int64_t GEMV_RUN_MAX_LDS = 65536;  // activation codes + scales held in LDS
bool gemv_run_supported(int64_t M, int64_t K, const void* x, const uint8_t* w_codes,
                        const uint8_t* w_scales);
hipError_t launch_gemv_run(const void* x, bool x_bf16, float* gsa, uint8_t* codes,
                           uint8_t* scales, const uint8_t* w_codes, const uint8_t* w_scales,
                           const float* ws2, void* y, bool y_bf16, int64_t M, int64_t N, int64_t K,
                           hipStream_t s);

// The narrow weight-streaming kernel handles these (4 weight rows per workgroup).
bool gemv_narrow_supported(int64_t M, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales);

bool gemv_narrow_run_supported(int64_t M, int64_t K, const void* x, const uint8_t* w_codes,
                               const uint8_t* w_scales);
hipError_t launch_narrow_run(const void* x, bool x_bf16, float* gsa, uint8_t* codes,
                             uint8_t* scales, const uint8_t* w_codes, const uint8_t* w_scales,
                             const float* ws2, void* y, bool y_bf16, int64_t M, int64_t N,
                             int64_t K, hipStream_t s);

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Grouped linear (or one projection: offsets NULL, G = 1) whose workgroups
// quantize their activation rows themselves from x (x_rows, K), bf16 or
// fp32, in ONE launch.  gsa: parts == NULL, from the amax of all of x, which
// every workgroup takes (keep x small); else from the maximum of the nparts
// partial maxima an earlier launch wrote (bits in x's format).  Workgroup
// (0, 0) writes gsa_out; codes_out / scales_out (or NULL) receive every row
// of x (parts == NULL) or the rows some group reads.  swiglu: the epilogue
// of nvfp4_grouped_linear_swiglu (y = h, partials_out gets one partial per
// workgroup, *nparts_out their count).  false from grouped_run_supported:
// not for these operands.
bool grouped_run_supported(int64_t x_rows, int64_t K, const void* x, const uint8_t* w_codes,
                           const uint8_t* w_scales);
hipError_t launch_grouped_run(const void* x, bool x_bf16, int64_t x_rows, const uint32_t* parts,
                              int64_t nparts, float* gsa_out, uint8_t* codes_out,
                              uint8_t* scales_out, const int32_t* row_index,
                              const int32_t* offsets, int G, int64_t M_total,
                              const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                              void* y, bool y_bf16, int64_t N, int64_t K, bool swiglu, int gran,
                              float limit, uint32_t* partials_out, int64_t* nparts_out,
                              hipStream_t s);

// The checks nvfp4_linear_run makes before any launch (an NVFP4_* status).
int linear_run_check(const void* x, int x_dtype, const float* gsa, const uint8_t* codes,
                     const uint8_t* scales, const uint8_t* w_codes, const uint8_t* w_scales,
                     const float* ws2, const void* y, int y_dtype, int64_t M, int64_t N,
                     int64_t K);

// Tiled GEMM for many rows (dequantize to f16, f16 matrix cores).
// Workspace for split K (fp32 partials) when the shape has few output tiles
// on the current device; 0 when it does not split.  Without it (ws NULL or
// smaller) launch_gemm runs unsplit.  With partial_splits, a split launch
// leaves its raw partial sums (split z at ws + z * M * N floats) for the
// caller to add and scale, and reports the split count there (0: y was
// written).
constexpr int GEMM_MAX_SPLITS = 16;
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                       void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s,
                       bool gsa_rows = false, void* ws = nullptr, size_t ws_bytes = 0,
                       int* partial_splits = nullptr);

// Grouped linear on the tiled GEMM (groups of many rows; arguments as
// launch_grouped_gemv).  Needs 16-byte aligned codes, 2-byte aligned
// scales, K % 256 == 0 and 32-bit code offsets of A and of one group's W.
constexpr int64_t GROUPED_MFMA_MIN_ROWS = 32;  // mean rows per group that take it
bool grouped_gemm_supported(const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* w_codes, const uint8_t* w_scales, int64_t a_rows,
                            int64_t M_total, int G, int64_t N, int64_t K);
hipError_t launch_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                               int64_t a_rows, const int32_t* row_index, const int32_t* offsets,
                               int G, int64_t M_total, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* ws2, void* y, bool y_bf16,
                               int64_t N, int64_t K, hipStream_t s);
// Workgroups (and so amax partials, with SwiGLU) of a grouped tiled launch.
int64_t grouped_tile_blocks(int64_t M_total, int G, int64_t N);
// The same with the SwiGLU epilogue of the gate/up projection (as
// launch_grouped_swiglu's kernel): h (M_total, N/2) fp32 and one partial per
// workgroup, grouped_tile_blocks of them.  N % (2 gran) == 0.
hipError_t launch_grouped_gemm_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                      const float* gsa, int64_t a_rows, const int32_t* row_index,
                                      const int32_t* offsets, int G, int64_t M_total,
                                      const uint8_t* w_codes, const uint8_t* w_scales,
                                      const float* ws2, float* h, int64_t N, int64_t K, int gran,
                                      float limit, uint32_t* partials, hipStream_t s);

}  // namespace nvfp4
