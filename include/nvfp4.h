/*
 * nvfp4.h -- C ABI of the NVFP4 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer runs in three steps on one GPU:
 *   1. amax -> gsa:  gsa = max(max_i |x_i|, 1e-8) / (6 * 448)
 *   2. quantize:     per 16-element block an E4M3 scale and 16 E2M1 codes
 *   3. linear:       y = gsa * ws2 * sum_k (lut[a]*sfa) * (lut[w]*sfw)
 * with a grouped form of step 3 for routed experts (and SwiGLU fused into
 * the gate/up projection), and around it the producer and consumers of the
 * same data: RMSNorm fused into steps 1-2, steps 1-2 on a weight at load
 * time, and the dense router's expert choice after a gate linear.
 *
 * Sources (pages of the nvfp4-megamoe-kernel repository on sweetapi.com):
 *   - commit 107d62d, single_shot_inference.py, commit message on computing
 *     gsa at runtime: gsa = max|x| / (6.0 * 448.0) keeps x/gsa <= 2688;
 *   - deleted PERFORMANCE_AUDIT.md, section "P0 -- Per-call .item() D2H
 *     sync": amax is clamped from below at 1e-8 and must stay on the GPU;
 *   - commit 107d62d, dsv4/ops/quantize.py, commit message: the amax is its
 *     own kernel (a single-pass kernel that synchronised only within a block
 *     raced across blocks), the quantize reads gsa from a device buffer;
 *   - commit 0d1cd1e, dsv4/kernels/indexer, commit message: E2M1 code table
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6} with bias 1, sign in bit 3;
 *   - commit db07d17, dsv4, commit messages: checkpoint weights are
 *     (N, K/2) uint8 (byte-identical to float4_e2m1fn_x2) with (N, K/16)
 *     E4M3 scales, and w = lut[w] * weight_scale * weight_scale_2;
 *   - dsv4/_archive/layers/linear.py (finalize_weights, _run_impl) and
 *     archived_plans/CORRECTNESS_BACKLOG.md section 7: the GEMM computes
 *     (A*SFA) @ (B*SFB) and the epilogue multiplies by gsa * gsb with
 *     gsb = weight_scale_2;
 *   - dsv4/_archive/layers/grouped_linear.py, _run_impl: one gsa shared by
 *     every group, one weight global scale per group;
 *   - README.md, "MoE kernel (FusedSwiGLUScaledGroupedGemmKernel)": L1
 *     gate/up weights interleaved at granularity 8, even subtiles gate, odd
 *     subtiles up, SwiGLU between the two expert projections.
 *
 * Data layout (all row-major, all buffers in device memory unless noted):
 *   x       (M, K) bf16 or fp32 activations; K % 16 == 0.
 *   codes   (M, K/2) uint8; byte j of a row holds element 2j in bits 0..3
 *           and element 2j+1 in bits 4..7; bit 3 of a code is its sign.
 *   scales  (M, K/16) uint8, E4M3 (OCP FP8 E4M3FN) bit patterns.
 *   gsa     one float32.
 *   weights codes (N, K/2) and scales (N, K/16), row n = output feature n;
 *           grouped weights are G such matrices stacked contiguously.
 *   ws2     one float32 per weight matrix (weight_scale_2).
 *   y       (M, N) float32 or bf16 (round to nearest even).
 *
 * Quantize rule for one 16-element block (binary32, correctly rounded):
 *   sf = E4M3_rne_satfinite(bamax / (gsa * 6));  s = dec(sf) * gsa;
 *   code = sign(x) | nearest_even_E2M1(|x| / s), magnitude 0 when sf == 0.
 *
 * Conventions:
 *   - The caller owns every buffer.  No entry point allocates, frees,
 *     synchronises or reads device memory on the host; all work is
 *     enqueued on `stream` (a hipStream_t; NULL is the null stream), so
 *     every call can be captured in a HIP graph.
 *   - Return value: NVFP4_OK (0) or a negative status; on any status other
 *     than NVFP4_ERR_LAUNCH nothing was enqueued.  nvfp4_status_string()
 *     names a status.
 *   - Stateless and reentrant; the workspace is scratch that the call may
 *     overwrite (its size comes from nvfp4_workspace_bytes; no initial
 *     contents are required, except nvfp4_router_topk's ticket counter,
 *     which must be zero before the first call and which every call leaves
 *     at zero).  Calls that share a workspace must be ordered on one
 *     stream.
 *   - Inputs must be finite.  A caller-supplied gsa must be positive and
 *     finite.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_OK 0
#define NVFP4_ERR_NULL (-1)      /* a required pointer is NULL            */
#define NVFP4_ERR_SHAPE (-2)     /* a size is negative, zero where it may  */
                                 /* not be, or K % 16 != 0                  */
#define NVFP4_ERR_DTYPE (-3)     /* unknown dtype enum                     */
#define NVFP4_ERR_WORKSPACE (-4) /* workspace NULL or smaller than needed  */
#define NVFP4_ERR_ALIGN (-5)     /* a pointer is not aligned as required   */
#define NVFP4_ERR_LAUNCH (-6)    /* the HIP runtime reported an error      */
#define NVFP4_ERR_SCRATCH (-7)   /* needs more than the static scratch     */

#define NVFP4_DTYPE_BF16 0
#define NVFP4_DTYPE_FP32 1

/* Operation ids for nvfp4_workspace_bytes. */
#define NVFP4_OP_AMAX_GSA 0
#define NVFP4_OP_QUANTIZE 1
#define NVFP4_OP_LINEAR 2
#define NVFP4_OP_GROUPED_LINEAR 3
#define NVFP4_OP_LINEAR_RUN 4
#define NVFP4_OP_GROUPED_SWIGLU 5
#define NVFP4_OP_QUANTIZE_WEIGHT 6
#define NVFP4_OP_RMSNORM_QUANTIZE 7
#define NVFP4_OP_ROUTER_TOPK 8
#define NVFP4_OP_GROUPED_RUN 9
#define NVFP4_OP_MOE_RUN 10

/* Bytes of workspace an operation needs for the given sizes (0 if none).
 * For NVFP4_OP_AMAX_GSA, M is the element count and N, K, G are ignored;
 * for NVFP4_OP_LINEAR_RUN, the activation is (M, K); for
 * NVFP4_OP_GROUPED_SWIGLU, M is M_total, N is N_inter and G the group count
 * (with M = 0 the size covers groups averaging fewer than 32 rows only);
 * for
 * NVFP4_OP_QUANTIZE_WEIGHT, the weight is (N, K); for
 * NVFP4_OP_RMSNORM_QUANTIZE, the activation is (M, K); for
 * NVFP4_OP_ROUTER_TOPK, M rows and N experts; for NVFP4_OP_GROUPED_RUN, x is
 * (M, K); for NVFP4_OP_MOE_RUN, M tokens, N = N1 and K = K1 of the first
 * projection and G experts (enough for up to M * G pairs: every token at
 * most once per expert; a call checks its own pair count). */
size_t nvfp4_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int G);

/* Step 1: gsa[0] = max(max_i |x_i|, 1e-8) / 2688.
 * x: numel elements of x_dtype (16-byte aligned); gsa: device float32.
 * A true grid reduction: the first kernel writes one partial maximum per
 * workgroup into ws, a second single-workgroup kernel reduces the partials
 * and writes gsa.  Inputs of at most 65536 elements are reduced by one
 * workgroup in a single kernel.  numel == 0 gives gsa = 1e-8 / 2688. */
int nvfp4_amax_gsa(const void *x, int x_dtype, int64_t numel, float *gsa, void *ws,
                   size_t ws_bytes, void *stream);

/* Step 2: quantize x (M, K) with the device gsa into codes (M, K/2) and
 * scales (M, K/16).  x 16-byte aligned, codes 8-byte aligned.  M == 0 is a
 * no-op.  gsa is read on the device; it need not come from step 1 (any
 * positive finite value works, a too small one saturates the scales at 448). */
int nvfp4_quantize_from_buffer(const void *x, int x_dtype, int64_t M, int64_t K,
                               const float *gsa, uint8_t *codes, uint8_t *scales,
                               void *stream);

/* Steps 1 and 2 in one call: gsa, codes (M, K/2) and scales (M, K/16) as
 * nvfp4_amax_gsa followed by nvfp4_quantize_from_buffer write them.  A
 * tensor of at most 16384 elements is done by ONE workgroup in one kernel
 * (its barrier spans every element, so the maximum is complete before any
 * block is quantized -- the cross-workgroup race of a single-pass kernel
 * that the pages record cannot occur); larger tensors run the amax as
 * nvfp4_amax_gsa does, then the quantize.  ws: nvfp4_workspace_bytes(
 * NVFP4_OP_AMAX_GSA, M * K, 0, 0, 0) bytes (0 up to 65536 elements).  x bf16 or fp32,
 * 16-byte aligned; codes 8-byte aligned; K % 16 == 0.  M == 0 writes
 * gsa = 1e-8 / 2688. */
int nvfp4_amax_quantize(const void *x, int x_dtype, int64_t M, int64_t K, float *gsa,
                        uint8_t *codes, uint8_t *scales, void *ws, size_t ws_bytes,
                        void *stream);

/* The producer of the activation fused into steps 1 and 2 (the pages' fused
 * RMSNorm + NVFP4 quantize feeding run_from_quantized with an optional
 * per-row gsa; the product form output = input * inv_rms * norm_weight from
 * archived_plans/CORRECTNESS_BACKLOG.md, "Compressor kv_norm", and
 * eps = 1e-6 from dsv4/_archive/layers/mhc.py): RMSNorm of each row of
 * x (M, K) with norm_weight (K,), inv_rms = 1 / sqrt(mean(x^2) + eps), then
 * steps 1 and 2 on the normalized rows -- without writing them out.
 * Two kernels (three with one global scale): one workgroup per row forms
 * inv_rms and the row's largest |y|, then the quantize recomputes y.
 *   - inv_rms (M,) float32 receives each row's scale.
 *   - The normalized value is y = (x * inv_rms) * w in float32 (two
 *     roundings, in that order), and y is what is quantized: codes (M, K/2),
 *     scales (M, K/16).
 *   - gsa_per_row == 0: one global scale, gsa[0] = max(max|y|, 1e-8) / 2688
 *     over the whole tensor (two-phase: row maxima into ws, then one
 *     workgroup reduces them); ws holds nvfp4_workspace_bytes(
 *     NVFP4_OP_RMSNORM_QUANTIZE, M, 0, K, 0) bytes.
 *   - gsa_per_row != 0: gsa (M,), gsa[m] from row m alone (then ws is not
 *     used); nvfp4_linear_rows takes such a gsa.
 * x and norm_weight bf16 or fp32, 16-byte aligned; K % 16 == 0; eps > 0
 * and finite (so a row of zeros normalizes to zeros, not 0 * inf).  The
 * mean of squares is a float32 sum, as a float32 RMSNorm forms it: a row
 * whose squares overflow float32 (|x| beyond about 1.8e19 / sqrt(K)) gets
 * inv_rms 0 and normalizes to zeros.
 * M == 0 writes gsa[0] = 1e-8 / 2688 (one scale) or nothing (per row). */
int nvfp4_rmsnorm_quantize(const void *x, int x_dtype, const void *norm_weight, int w_dtype,
                           float eps, int64_t M, int64_t K, int gsa_per_row, float *gsa,
                           float *inv_rms, uint8_t *codes, uint8_t *scales, void *ws,
                           size_t ws_bytes, void *stream);

/* Weight-side quantize at load time (the pages' quantize_weight_to_nvfp4 for the lm_head and router gate, whose
 * checkpoints hold bf16): w (N, K) bf16/fp32, K % 16 == 0, 16-byte
 * aligned, becomes codes (N, K/2), scales (N, K/16) and its global scale
 * ws2[0] = max(max|w|, 1e-8) / 2688 -- the activation recipe of steps 1
 * and 2 applied to the weight, with the result in the layout nvfp4_linear
 * takes, and the same results as nvfp4_amax_gsa + nvfp4_quantize_from_buffer
 * on w.  ws: nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE_WEIGHT, 0, N, K, 0)
 * bytes (the amax partials). */
int nvfp4_quantize_weight(const void *w, int w_dtype, int64_t N, int64_t K, float *ws2,
                          uint8_t *codes, uint8_t *scales, void *ws, size_t ws_bytes,
                          void *stream);

/* Step 3: y (M, N) = gsa * ws2 * dequant(A) @ dequant(W)^T, FP32 accumulation.
 * A is codes (M, K/2) + scales (M, K/16) from step 2; W is codes (N, K/2) +
 * scales (N, K/16); gsa and ws2 are device float32 scalars.  Code buffers
 * 8-byte aligned.  M <= 16 runs a weight-streaming kernel on FP4 matrix
 * cores (with 16-byte aligned operands and K % 256 == 0, the weight ring of
 * nvfp4_grouped_linear for 1-2 rows from N = 8192 and 3-4 rows from 10240,
 * and the tiled kernel, unsplit, for 8-16 rows from N = 10240, 15-16 rows
 * from 6144 and 5-16 rows from 16384, where those measured faster); larger
 * M runs a tiled kernel that dequantizes both operands exactly to f16
 * (every E2M1 x E4M3 product fits) and accumulates on f16 matrix cores in
 * FP32.  M == 0 or N == 0 is a no-op.
 * ws is optional.  With few output tiles (a 128 x 64 tile each; at most
 * half as many tiles as the device has compute units) and K a multiple of
 * 256 the tiled kernel can split K across workgroups: each split writes its
 * fp32 partial sums into ws and a second kernel adds them in split order
 * (deterministic) and applies the epilogue.  That needs
 * nvfp4_workspace_bytes(NVFP4_OP_LINEAR, M, N, K, 0) bytes (0 when the
 * shape does not split on the current device), 16-byte aligned; with a
 * NULL or smaller ws the kernel runs unsplit, with the same results up to
 * the fp32 summation order. */
int nvfp4_linear(const uint8_t *a_codes, const uint8_t *a_scales, const float *gsa,
                 const uint8_t *w_codes, const uint8_t *w_scales, const float *ws2,
                 void *y, int y_dtype, int64_t M, int64_t N, int64_t K, void *ws,
                 size_t ws_bytes, void *stream);

/* Step 3 with one activation global scale per row (the optional per-row gsa
 * of the pages' run_from_quantized): as nvfp4_linear, but gsa_rows is a
 * device float32[M] and y[m] = gsa_rows[m] * ws2 * dequant(A[m]) @
 * dequant(W)^T -- the product nvfp4_rmsnorm_quantize(..., gsa_per_row = 1)
 * feeds.  Same kernels, checks, alignment and optional split-K workspace
 * as nvfp4_linear; the epilogue multiplies by gsa_rows[m] * ws2 in
 * float32.  M == 0 or N == 0 is a no-op. */
int nvfp4_linear_rows(const uint8_t *a_codes, const uint8_t *a_scales, const float *gsa_rows,
                      const uint8_t *w_codes, const uint8_t *w_scales, const float *ws2,
                      void *y, int y_dtype, int64_t M, int64_t N, int64_t K, void *ws,
                      size_t ws_bytes, void *stream);

/* The dense router's gate projection and expert choice (the pages'
 * "Dense Router": sqrt(softplus(X @ W_gate)) + e_bias and top-k selection,
 * archived_plans/CORRECTNESS_BACKLOG.md section 5; the gsa * gsb factor on
 * the logit before sqrt(softplus) from the router gate commit message of
 * single_shot_inference.py, commit 107d62d; shipped there as the NVFP4 GEMM
 * followed by an activation + top-k kernel).
 *   logit[m, j] = gsa * ws2 * dequant(A[m]) . dequant(W[j])   (step 3; W is
 *                 the gate weight, one row per expert, e.g. quantized at
 *                 load time by nvfp4_quantize_weight)
 *   s[m, j]     = sqrt(softplus(logit[m, j])),  softplus(z) = log(1 + e^z)
 *   v[m, j]     = s[m, j] + bias[j]             (bias (N,) fp32, or NULL: 0)
 * topk_idx (M, topk) int32 receives the topk experts of largest v, best
 * first, the lower expert index first among equal v; topk_score (M, topk)
 * fp32 receives their s (the bias steers the choice only).  The scores are
 * float32: softplus and sqrt from the device math library (a few ulp).
 * N <= 1024 experts; 1 <= topk <= min(N, 64); other checks as nvfp4_linear.
 * ws: nvfp4_workspace_bytes(NVFP4_OP_ROUTER_TOPK, M, N, K, 0) bytes,
 * 16-byte aligned; on return it starts with the fp32 logits (M, N)
 * row-major.  What follows them (from byte L = M * N * 4 rounded up to 16):
 *   - M <= 16: ONE kernel (the pages' single-kernel gate GEMM with the
 *     sqrt(softplus) + bias + top-k epilogue, commit db07d17's message).
 *     The weight-streaming linear's workgroups write the logits with
 *     device-coherent (agent-scope atomic) stores and wait for them; each
 *     then takes a ticket from a counter, the uint32 at byte L (a
 *     device-scope atomic add), and the workgroup with the last ticket reads
 *     the logits with device-coherent loads, chooses the experts of every
 *     row and sets the counter back to zero.
 *     No workgroup waits for another.  That word must be ZERO before the
 *     first call with a given workspace (allocate it zeroed); every call
 *     leaves it zero.  Calls that share a workspace must be ordered.
 *   - M > 16: the linear's split-K partials; two kernels, the linear and
 *     one wave per row for the activation, bias and choice (which also adds
 *     the split-K partials).
 * M == 0 is a no-op. */
int nvfp4_router_topk(const uint8_t *a_codes, const uint8_t *a_scales, const float *gsa,
                      const uint8_t *w_codes, const uint8_t *w_scales, const float *ws2,
                      const float *bias, int64_t M, int64_t N, int64_t K, int topk,
                      int32_t *topk_idx, float *topk_score, void *ws, size_t ws_bytes,
                      void *stream);

/* The whole layer on a bf16/fp32 activation, as Nvfp4Linear.run does
 * (dsv4/_archive/layers/linear.py, _run_impl): steps 1, 2 and 3 with the
 * same results as calling nvfp4_amax_gsa, nvfp4_quantize_from_buffer and
 * nvfp4_linear in turn -- gsa, codes (M, K/2) and scales (M, K/16) are
 * written as those calls would write them, and y (M, N).
 * When x, w_codes and w_scales are 16-byte aligned it is ONE kernel for
 *   - up to 2 rows with N >= 24576, K % 256 == 0 and M*K <= 16384 (the
 *     weight-streaming ring of nvfp4_grouped_linear_run, 128 weight rows per
 *     workgroup: a long weight stream such as the lm_head's), or, where
 *     nvfp4_linear would not take its ring or tiles for the shape (one row
 *     below N = 12288 excepted; the others run steps 1-2, then that path),
 *   - up to 4 rows with K % 512 == 0, K <= 16384 and M*K <= 16384 (8 weight
 *     rows per workgroup), or
 *   - up to 16 rows with K % 256 == 0, M*K/16 <= 1024 and
 *     M*(K/2 + K/16) <= 65536 (16 weight rows per workgroup):
 * every workgroup reads the whole activation, computes its exact maximum by
 * itself (no reduction across workgroups, so no workgroup waits on
 * another), quantizes it into LDS and streams its weight rows; workgroup 0
 * also writes gsa, codes and scales.  Otherwise steps 1-2 run as
 * nvfp4_amax_quantize does (one kernel up to 16384 elements), then step 3
 * (ws must hold nvfp4_workspace_bytes(NVFP4_OP_LINEAR_RUN, M, N, K, 1)
 * bytes: the amax partials, and after them the optional split K of
 * nvfp4_linear).
 * N == 0 only quantizes. */
int nvfp4_linear_run(const void *x, int x_dtype, float *gsa, uint8_t *codes, uint8_t *scales,
                     const uint8_t *w_codes, const uint8_t *w_scales, const float *ws2, void *y,
                     int y_dtype, int64_t M, int64_t N, int64_t K, void *ws, size_t ws_bytes,
                     void *stream);

/* nvfp4_linear_run for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks, kernels and results, without the
 * workspace.  Its scratch (the amax partials and the linear's split-K
 * partials) is a device array of NVFP4_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; the call allocates
 * nothing and calls no allocating routine.  A shape whose workspace,
 * nvfp4_workspace_bytes(NVFP4_OP_LINEAR_RUN, M, N, K, 1), exceeds that size
 * returns NVFP4_ERR_SCRATCH and launches nothing.  Every call on one GPU
 * shares the array: calls that overlap on a GPU (other streams, other
 * threads) race and must be ordered by the caller.  The stream must belong
 * to the calling thread's current device. */
#define NVFP4_NOALLOC_SCRATCH_BYTES (16u << 20)
int nvfp4_linear_run_noalloc(const void *x, int x_dtype, float *gsa, uint8_t *codes,
                             uint8_t *scales, const uint8_t *w_codes, const uint8_t *w_scales,
                             const float *ws2, void *y, int y_dtype, int64_t M, int64_t N,
                             int64_t K, void *stream);

/* Grouped linear (MoE experts, or any set of G weight matrices sharing one
 * activation gsa).  Output row r, 0 <= r < M_total, belongs to group g when
 * group_offsets[g] <= r < group_offsets[g+1] (device int32[G+1],
 * non-decreasing); its activation row is row_index[r] (device
 * int32[M_total]) or r when row_index is NULL (then a_rows >= M_total).
 * A has a_rows rows (codes (a_rows, K/2), scales (a_rows, K/16)).
 * y[r] = gsa * ws2[g] * dequant(A[row]) @ dequant(W_g)^T with W_g = codes
 * (N, K/2) at w_codes + g*N*K/2 and scales (N, K/16) at w_scales + g*N*K/16;
 * ws2 is a device float32[G].  The group sizes are read on the device only.
 * Rows of y outside every group, rows at or beyond M_total, and rows whose
 * row_index lies outside [0, a_rows) are not written.  group_offsets must
 * be non-decreasing; rows of groups that break that may be left unwritten.
 * Kernels: with at least 32 rows per group on average (M_total / G), 16-byte
 * aligned codes, 2-byte aligned scales and K % 256 == 0, one launch of
 * 64 x 128 output tiles over every group's rows on the f16 matrix cores
 * (the pages' grouped block-scaled GEMM); otherwise one launch that streams
 * each group's weights once per 8 or 16 of its rows. */
int nvfp4_grouped_linear(const uint8_t *a_codes, const uint8_t *a_scales, const float *gsa,
                         int64_t a_rows, const int32_t *row_index,
                         const int32_t *group_offsets, int G, int64_t M_total,
                         const uint8_t *w_codes, const uint8_t *w_scales, const float *ws2,
                         void *y, int y_dtype, int64_t N, int64_t K, void *stream);

/* The grouped linear on a bf16/fp32 activation, steps 1-3 in as few
 * launches as the sizes allow (the decode of G weight matrices that share
 * one activation's global scale: the pages' dense grouped linear for wo_a,
 * where token t's slice for group g is row t*G + g of x -- or the routed
 * experts of a decoded token).  Same results as
 *   nvfp4_amax_quantize(x (x_rows, K)) -> gsa, x_codes, x_scales
 *   nvfp4_grouped_linear(x_codes, x_scales, gsa, x_rows, row_index, ...)
 * (dsv4/_archive/layers/grouped_linear.py, _run_impl: one gsa over the whole
 * activation, then the grouped GEMM; README.md's MoE kernel section for the
 * routed case).  gsa, x_codes (x_rows, K/2) and x_scales (x_rows, K/16)
 * are written as those calls write them, except that rows of x no output
 * row reads may be left unwritten when x has more than 16384 elements.
 * When x, w_codes and w_scales are 16-byte aligned and K % 256 == 0:
 *   - x of at most 16384 elements: ONE launch.  Every workgroup reduces all
 *     of x itself (so none waits on another), forms gsa, quantizes the rows
 *     it reads into its LDS and streams its weight tiles;
 *   - larger x: two launches, the amax partials (ws) and then the grouped
 *     linear, every workgroup of which reduces the partials itself.
 * Otherwise the two calls above.  ws: nvfp4_workspace_bytes(
 * NVFP4_OP_GROUPED_RUN, x_rows, N, K, G) bytes (0 for the one-launch case),
 * 4-byte aligned.  Row conventions and other checks as nvfp4_grouped_linear
 * (x_codes 8-byte aligned).  x_rows == 0 writes gsa = 1e-8 / 2688 and
 * needs M_total == 0 or N == 0. */
int nvfp4_grouped_linear_run(const void *x, int x_dtype, int64_t x_rows, float *gsa,
                             uint8_t *x_codes, uint8_t *x_scales, const int32_t *row_index,
                             const int32_t *group_offsets, int G, int64_t M_total,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *ws2,
                             void *y, int y_dtype, int64_t N, int64_t K, void *ws,
                             size_t ws_bytes, void *stream);

/* The routed-expert pair on a bf16/fp32 activation x (T, K1), the pages'
 * Nvfp4MoE (README.md, "MoE kernel": granularity-interleaved gate/up first
 * projection, SwiGLU, second projection; dsv4/ops/quantize.py's commit
 * message on the fused de-interleave + amax + quantize between them).  Same
 * results as
 *   nvfp4_amax_quantize(x) -> gsa_x, x_codes (T, K1/2), x_scales (T, K1/16)
 *   nvfp4_grouped_linear_swiglu(x_codes, ..., row_index, group_offsets, E, P,
 *       w1 (E, N1, K1), ..., h (P, N1/2), gsa_h, h_codes, h_scales, ...)
 *   nvfp4_grouped_linear(h_codes, h_scales, gsa_h, P, NULL, group_offsets,
 *       E, P, w2 (E, N2, N1/2), ..., y (P, N2))
 * with the same rules for rows outside every group (h and y are written
 * only for rows some expert reads, and h's amax covers only those rows;
 * when h is quantized by a launch of its own, h_codes and h_scales are
 * written for every row, from whatever h holds in the others).  Launches:
 *   - the first projection, whose workgroups quantize x themselves when x
 *     has at most 16384 elements (a decoded token); else x's amax and
 *     quantize come first (one or two launches);
 *   - the second projection, whose workgroups reduce the first's amax
 *     partials and quantize the rows of h they read themselves, when the
 *     first projection had at most 2048 workgroups and the experts average
 *     fewer than 32 pairs; else h's finalize and quantize come first.
 * With 32 pairs or more per expert on average both projections run on the
 * 64 x 128 tiles of nvfp4_grouped_linear.  One decoded token routed to 8
 * experts is two launches.
 * Requires row_index (token of each pair), granularity 1, 2, 4 or 8,
 * N1 % (2 granularity) == 0, K1 and N1/2 multiples of 256 (short enough to
 * stage), and every buffer but y and the scalars 16-byte aligned.
 * ws: nvfp4_workspace_bytes(NVFP4_OP_MOE_RUN, T, N1, K1, E) bytes.
 * limit: the SwiGLU limit, as in nvfp4_swiglu_deinterleave.  P == 0 only
 * quantizes x and writes gsa_h = 1e-8 / 2688. */
int nvfp4_moe_run(const void *x, int x_dtype, int64_t T, float *gsa_x, uint8_t *x_codes,
                  uint8_t *x_scales, const int32_t *row_index, const int32_t *group_offsets,
                  int E, int64_t P, const uint8_t *w1_codes, const uint8_t *w1_scales,
                  const float *w1_ws2, int64_t N1, int64_t K1, int granularity, float limit,
                  float *h, float *gsa_h, uint8_t *h_codes, uint8_t *h_scales,
                  const uint8_t *w2_codes, const uint8_t *w2_scales, const float *w2_ws2,
                  int64_t N2, void *y, int y_dtype, void *ws, size_t ws_bytes, void *stream);

/* SwiGLU between the two expert projections, unfused: l1 (M, N_inter) fp32
 * holds gate/up column groups of `granularity` columns interleaved (group
 * q = j / granularity is gate when q is even, up when odd, gate group 2p
 * pairs with up group 2p+1); h (M, N_inter/2) fp32 receives
 * h[m, p*granularity + i] = silu(gate) * up, silu(g) = g / (1 + exp(-g)).
 * N_inter % (2*granularity) == 0.
 * limit: <= 0 applies none.  > 0 first caps the gate at limit and clamps the
 * up value to [-limit, limit] (archived_plans/CORRECTNESS_BACKLOG.md
 * section 6, Nvfp4MoE, lists a SwiGLU limit of 10 without its formula; this
 * clamp is the reading taken).  NaN: NVFP4_ERR_SHAPE. */
int nvfp4_swiglu_deinterleave(const float *l1, float *h, int64_t M, int64_t N_inter,
                              int granularity, float limit, void *stream);

/* The step between the two expert projections, fused into the first
 * (SwiGLU, de-interleave and the first amax phase in the grouped gate/up
 * linear's epilogue; the pages' fused SwiGLU
 * grouped GEMM epilogue, and the de-interleave + amax + quantize kernel that
 * consumes its output).  Same results as
 *   nvfp4_grouped_linear(..., l1, FP32, N_inter, K, ...)   l1 (M_total, N_inter)
 *   nvfp4_swiglu_deinterleave(l1, h, M_total, N_inter, granularity)
 *   nvfp4_amax_gsa(h, FP32, M_total * N_inter / 2, gsa_h, ...)
 * without the fp32 l1: h (M_total, N_inter/2) fp32 and gsa_h (device
 * float32[1]) are written, h bit-identical to the unfused calls.  Rows of
 * h that nvfp4_grouped_linear would leave unwritten (outside every group,
 * or whose row_index lies outside [0, a_rows)) are not written and do not
 * enter the amax.  The amax is a two-phase grid reduction: every workgroup
 * of the linear writes the largest |h| it wrote into ws, and a second
 * kernel reduces those and writes gsa_h.  The linear is the weight ring
 * for few rows per group, or with 32 rows or more per group on average the
 * 64 x 128 tiles of nvfp4_grouped_linear (the same kernels the unfused
 * call takes, so h stays bit-identical).
 * Requires granularity 1, 2, 4 or 8 (a wave's 16 output columns, and a
 * tile's 128, then hold whole gate/up pairs), N_inter % (2*granularity) == 0, K % 256 == 0, K
 * short enough for the staged kernel (K <= 48 384), a_rows*K/2 < 2^31, and
 * 16-byte aligned codes and scales (NVFP4_ERR_SHAPE / NVFP4_ERR_ALIGN
 * otherwise; then call the three functions above).
 * ws: nvfp4_workspace_bytes(NVFP4_OP_GROUPED_SWIGLU, M_total, N_inter, 0, G)
 * bytes, 4-byte aligned, overwritten.
 * h_codes (M_total, N_inter/4) and h_scales (M_total, N_inter/32), both or
 * neither (NULL): also step 2 on h with gsa_h, as
 *   nvfp4_quantize_from_buffer(h, FP32, M_total, N_inter/2, gsa_h, ...)
 * writes it -- every row of h, including rows left unwritten above (they
 * carry whatever h held) -- the pages' fused de-interleave + amax +
 * quantize.  With at most 2048 amax partials each quantize workgroup
 * reduces them itself, so the second amax phase and the quantize are one
 * kernel.  Needs (N_inter/2) % 16 == 0; h_codes 8-byte aligned and h
 * 16-byte aligned.
 * limit: the SwiGLU limit, as in nvfp4_swiglu_deinterleave.
 * M_total == 0 or N_inter == 0 only writes gsa_h (the 1e-8 floor). */
int nvfp4_grouped_linear_swiglu(const uint8_t *a_codes, const uint8_t *a_scales,
                                const float *gsa, int64_t a_rows, const int32_t *row_index,
                                const int32_t *group_offsets, int G, int64_t M_total,
                                const uint8_t *w_codes, const uint8_t *w_scales,
                                const float *ws2, float *h, float *gsa_h, uint8_t *h_codes,
                                uint8_t *h_scales, int64_t N_inter, int64_t K, int granularity,
                                float limit, void *ws, size_t ws_bytes, void *stream);

/* Static name of a status code. */
const char *nvfp4_status_string(int status);

/* Library ABI version (increments when an entry point is added or a
 * signature changes). */
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
