/*
 * nvfp4_oracle.c -- plain, slow CPU definition of the NVFP4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it (through oracle/oracle.py).  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Sources (pages of the nvfp4-megamoe-kernel repository on sweetapi.com):
 *   [E2M1]  commit 0d1cd1e, dsv4/kernels/indexer: commit message on the E2M1
 *           decode fix (the bias-1 encoding table and the wrong "raw integer"
 *           decode it replaced).
 *   [GSA]   commit 107d62d, single_shot_inference.py: commit message "compute
 *           gsa at runtime from actual activation magnitude" (max|x|/(6*448)).
 *   [AMAX]  deleted PERFORMANCE_AUDIT.md, section "P0 -- Per-call .item()
 *           D2H sync" (amax clamped from below at 1e-8, then /(6*448)).
 *   [TWOK]  commit 107d62d, dsv4/ops/quantize.py: commit message on the
 *           cross-CTA amax race (amax kernel, then quantize from a buffer).
 *   [WS2]   commit db07d17, dsv4: commit message "weight_scale_2 was being
 *           dropped" (w = lut[w] * weight_scale * weight_scale_2).
 *   [LIN]   dsv4/_archive/layers/linear.py, finalize_weights comment
 *           (y = (x*scale_a*gsa) @ (w*scale_b*gsb)).
 *   [CB7]   archived_plans/CORRECTNESS_BACKLOG.md, section 7 "NVFP4
 *           Quantization" (gsb = weight_scale_2; E4M3 max 448, FP4 max 6).
 *   [GL]    dsv4/_archive/layers/grouped_linear.py, _run_impl (one gsa shared
 *           by every group; each group has its own weight global scale).
 *   [MOE]   README.md, "MoE kernel (FusedSwiGLUScaledGroupedGemmKernel)":
 *           granularity-8 interleaved L1 weights, even subtiles gate, odd up.
 *   [NORM]  archived_plans/CORRECTNESS_BACKLOG.md, "Compressor kv_norm --
 *           VERIFIED CORRECT" (output = input * inv_rms * norm_weight[c]);
 *           dsv4/_archive/layers/mhc.py, module constants (EPS_RMSN = 1e-6).
 *   [ROUTE] archived_plans/CORRECTNESS_BACKLOG.md, section 5 "Router",
 *           "Dense Router" (expert scores sqrt(softplus(X @ W_gate)) plus
 *           e_bias, then top-k selection); commit 107d62d,
 *           single_shot_inference.py, commit message on the router gate's
 *           global scales (the epilogue applies gsa * gsb to the logit
 *           before sqrt(softplus)).
 *
 * Where the pages are silent, each function below states the reading it
 * takes.
 *
 * Floating point: every float operation is a single IEEE binary32 operation,
 * correctly rounded (build with -O2 -fno-fast-math -ffp-contract=off), in
 * the order written.  GEMM sums are taken in binary64 in ascending k.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#include <omp.h>

#define ORACLE_BF16 0
#define ORACLE_FP32 1

/* ------------------------------------------------------------------ */
/* E2M1: sign bit 3, exponent bits 2..1, mantissa bit 0, exponent bias 1.
 * exp 0 is subnormal (0 or 0.5); exp e>0 is 2^(e-1) * (1 + m/2).  [E2M1]
 * Decoded from the bit fields, not from a table, so that the table printed
 * on the page is an independent check of this function. */
double oracle_e2m1_value(unsigned code)
{
    unsigned sign = (code >> 3) & 1u;
    unsigned e = (code >> 1) & 3u;
    unsigned m = code & 1u;
    double mag;
    if (e == 0)
        mag = 0.5 * (double)m;
    else
        mag = ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return sign ? -mag : mag;
}

/* Nearest E2M1 magnitude index (0..7) to q >= 0, ties to the code whose
 * mantissa bit is 0 (round half to even), values beyond 6 go to 6
 * (saturation).  Brute force over the eight grid points. */
unsigned oracle_e2m1_nearest(float q)
{
    if (q >= 6.0f)
        return 7; /* at or beyond the largest magnitude (huge q would tie in double) */
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
        double d = fabs((double)q - oracle_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1u) == 0u)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* E4M3 (OCP FP8 E4M3FN): sign bit 7, exponent bits 6..3 (bias 7), mantissa
 * bits 2..0; exponent field 0 is subnormal (m * 2^-9); 0x7F/0xFF are NaN and
 * there is no infinity, so the largest finite value is 0x7E = 448. [CB7] */
double oracle_e4m3_value(unsigned byte)
{
    unsigned sign = (byte >> 7) & 1u;
    unsigned e = (byte >> 3) & 15u;
    unsigned m = byte & 7u;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return sign ? -mag : mag;
}

/* Encode v >= 0 to the nearest non-negative finite E4M3 value, ties to the
 * even code (mantissa LSB 0), anything above 448 to 448 (saturate to the
 * largest finite value).  Brute force over all 127 finite codes. */
unsigned oracle_e4m3_encode(float v)
{
    if (v >= 448.0f)
        return 0x7E; /* at or beyond the largest finite value */
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c < 0x7F; ++c) {
        double d = fabs((double)v - oracle_e4m3_value(c));
        if (d < bestd || (d == bestd && (c & 1u) == 0u)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ */
static float load_elem(const void *x, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16) {
        uint16_t h = ((const uint16_t *)x)[i];
        uint32_t u = (uint32_t)h << 16; /* bf16 -> fp32 is exact */
        float f;
        memcpy(&f, &u, 4);
        return f;
    }
    return ((const float *)x)[i];
}

/* amax = max_i |x_i|  (exact; the max of absolute values). [GSA] [AMAX] */
float oracle_amax(const void *x, int dtype, int64_t n)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(load_elem(x, dtype, i));
        if (a > amax)
            amax = a;
    }
    return amax;
}

/* gsa = max(amax, 1e-8) / (6 * 448), the divisor taken as the exact 2688.
 * [AMAX] clamp, [GSA] formula.  The page's expression is evaluated in double
 * then stored as float32; one binary32 division gives the same value because
 * a double-rounded quotient is innocuous at 53 >= 2*24+2 bits. */
float oracle_gsa(float amax)
{
    if (!(amax >= 1e-8f))
        amax = 1e-8f;
    return amax / 2688.0f;
}

/* Quantize an M x K row-major tensor (K % 16 == 0) with a given gsa.
 * For each row m and 16-element block b:
 *   bamax  = max |x| over the block
 *   sf     = E4M3(bamax / (gsa * 6))        (RNE, satfinite)
 *   s      = dec(sf) * gsa
 *   code_k = sign(x_k) | nearest_E2M1(|x_k| / s)   (0 if dec(sf) == 0)
 * codes: M x K/2 bytes, byte j of a row holds element 2j in bits 0..3 and
 * element 2j+1 in bits 4..7.  scales: M x K/16 bytes.
 * The block-scale formula (map the block maximum onto the largest E2M1
 * magnitude 6) and dividing by the rounded scale are this oracle's reading;
 * the pages give only gsa and the dequant rule [WS2] [LIN]. */
void oracle_quantize(const void *x, int dtype, int64_t M, int64_t K, float gsa,
                     uint8_t *codes, uint8_t *scales)
{
    int64_t nb = K / 16;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            float v[16];
            float bamax = 0.0f;
            for (int j = 0; j < 16; ++j) {
                v[j] = load_elem(x, dtype, m * K + b * 16 + j);
                if (fabsf(v[j]) > bamax)
                    bamax = fabsf(v[j]);
            }
            float six_gsa = gsa * 6.0f;
            float sf_raw = bamax / six_gsa;
            unsigned sf = oracle_e4m3_encode(sf_raw);
            scales[m * nb + b] = (uint8_t)sf;
            float sdec = (float)oracle_e4m3_value(sf); /* exact in float */
            float s = sdec * gsa;
            for (int j = 0; j < 16; ++j) {
                unsigned mag = 0;
                if (sdec != 0.0f) {
                    float q = fabsf(v[j]) / s;
                    mag = oracle_e2m1_nearest(q);
                }
                unsigned code = (signbit(v[j]) ? 8u : 0u) | mag;
                int64_t k = b * 16 + j;
                uint8_t *byte = &codes[m * (K / 2) + k / 2];
                if ((k & 1) == 0)
                    *byte = (uint8_t)((*byte & 0xF0u) | code);
                else
                    *byte = (uint8_t)((*byte & 0x0Fu) | (code << 4));
            }
        }
    }
}

/* Dequantized element value lut[code] * dec(sf) (exact in double); the
 * global scale is applied separately.  [WS2] */
static double deq(const uint8_t *codes, const uint8_t *scales, int64_t K,
                  int64_t row, int64_t k)
{
    uint8_t byte = codes[row * (K / 2) + k / 2];
    unsigned code = (k & 1) ? (byte >> 4) : (byte & 0x0Fu);
    return oracle_e2m1_value(code) * oracle_e4m3_value(scales[row * (K / 16) + k / 16]);
}

/* x_hat = lut[code] * dec(sf) * gsa, as double (M x K). */
void oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float gsa,
                       int64_t M, int64_t K, double *out)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            out[m * K + k] = deq(codes, scales, K, m, k) * (double)gsa;
}

/* One output of the linear layer:
 *   y[m,n] = gsa * ws2 * sum_k (lut[a]*sfa) * (lut[w]*sfw)
 * every term exact in double, summed in ascending k.  [LIN] [WS2] [CB7] */
static double dot_row(const uint8_t *a_codes, const uint8_t *a_scales, int64_t arow,
                      const uint8_t *w_codes, const uint8_t *w_scales, int64_t wrow,
                      int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += deq(a_codes, a_scales, K, arow, k) * deq(w_codes, w_scales, K, wrow, k);
    return acc;
}

/* y (M x N, double) = gsa * ws2 * A_hat @ W_hat^T ; W is N x K (row n = output n). */
void oracle_linear(const uint8_t *a_codes, const uint8_t *a_scales, float gsa,
                   const uint8_t *w_codes, const uint8_t *w_scales, float ws2,
                   int64_t M, int64_t N, int64_t K, double *y)
{
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < M * N; ++i) {
        int64_t m = i / N, n = i % N;
        y[i] = (double)gsa * (double)ws2 * dot_row(a_codes, a_scales, m, w_codes, w_scales, n, K);
    }
}

/* The same outputs at a list of (m, n) positions only. */
void oracle_linear_at(const uint8_t *a_codes, const uint8_t *a_scales, float gsa,
                      const uint8_t *w_codes, const uint8_t *w_scales, float ws2,
                      int64_t K, int64_t npos, const int64_t *ms, const int64_t *ns,
                      double *y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npos; ++i)
        y[i] = (double)gsa * (double)ws2 *
               dot_row(a_codes, a_scales, ms[i], w_codes, w_scales, ns[i], K);
}

/* Grouped linear.  Output row r belongs to group g when
 * offsets[g] <= r < offsets[g+1]; its activation row is row_index[r] (or r
 * when row_index is NULL).  Group g has its own weights (N x K codes and
 * N x K/16 scales at offset g in the stacked arrays) and its own ws2[g]; one
 * gsa is shared by all groups.  [GL] [WS2]  Rows outside every group are not
 * written. */
void oracle_grouped_linear(const uint8_t *a_codes, const uint8_t *a_scales, float gsa,
                           const int32_t *row_index, const int32_t *offsets, int G,
                           const uint8_t *w_codes, const uint8_t *w_scales,
                           const float *ws2, int64_t N, int64_t K, double *y)
{
    for (int g = 0; g < G; ++g) {
        const uint8_t *wc = w_codes + (int64_t)g * N * (K / 2);
        const uint8_t *ws = w_scales + (int64_t)g * N * (K / 16);
        int64_t r0 = offsets[g], r1 = offsets[g + 1];
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = r0; r < r1; ++r) {
            int64_t arow = row_index ? row_index[r] : r;
            for (int64_t n = 0; n < N; ++n)
                y[r * N + n] = (double)gsa * (double)ws2[g] *
                               dot_row(a_codes, a_scales, arow, wc, ws, n, K);
        }
    }
}

/* Column j of the interleaved gate/up output belongs to group q = j / gran;
 * even q are gate columns and odd q up columns, pairing gate group q with
 * up group q+1 [MOE].  h[:, (q/2)*gran + j%gran] = silu(gate) * up with
 * silu(g) = g / (1 + exp(-g)), in double.
 * limit > 0: the pages name a SwiGLU limit (10 for the model) without its
 * formula; the reading taken here caps the gate from above,
 * g = min(g, limit), and clamps the up value to [-limit, limit] before the
 * product.  limit <= 0: no clamp. */
void oracle_swiglu_deinterleave(const float *l1, int64_t M, int64_t N_inter,
                                int gran, double limit, double *h)
{
    int64_t H = N_inter / 2;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < H; ++c) {
            int64_t pair = c / gran, off = c % gran;
            double g = l1[m * N_inter + (2 * pair) * gran + off];
            double u = l1[m * N_inter + (2 * pair + 1) * gran + off];
            if (limit > 0.0) {
                g = fmin(g, limit);
                u = fmin(fmax(u, -limit), limit);
            }
            h[m * H + c] = g / (1.0 + exp(-g)) * u;
        }
    }
}

/* RMSNorm of each row [NORM]: inv_rms[m] = 1 / sqrt(mean_k x[m,k]^2 + eps)
 * and y[m,k] = x[m,k] * inv_rms[m] * w[k], all in binary64 (the sum of
 * squares in ascending k).  The pages give the product form and the eps;
 * eps is added to the mean of the squares (the usual RMSNorm; a variant
 * on the pages adds it to the sum instead, which this does not take).
 * y may be NULL. */
void oracle_rmsnorm(const void *x, int x_dtype, const void *w, int w_dtype, double eps,
                    int64_t M, int64_t K, double *inv_rms, double *y)
{
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)load_elem(x, x_dtype, m * K + k);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        inv_rms[m] = r;
        if (y)
            for (int64_t k = 0; k < K; ++k)
                y[m * K + k] = (double)load_elem(x, x_dtype, m * K + k) * r *
                               (double)load_elem(w, w_dtype, k);
    }
}

/* Router scores [ROUTE], in binary64: for each logit z (the linear's output,
 * gsa * gsb already applied), s = sqrt(softplus(z)) with
 * softplus(z) = log(1 + exp(z)) written as max(z, 0) + log1p(exp(-|z|)),
 * which is the same function without overflow for large |z|. */
void oracle_router_scores(const double *logits, int64_t n, double *s)
{
    for (int64_t i = 0; i < n; ++i) {
        double z = logits[i];
        double sp = (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
        s[i] = sqrt(sp);
    }
}

/* Top-k routing [ROUTE]: per row of logits (M, N), v_j = s_j + bias_j
 * (bias may be NULL: zero), and the k experts of largest v are chosen, best
 * first.  The pages do not order equal values; the reading taken is the
 * lower expert index first.  The bias only steers the choice: score[r] is
 * s (without the bias) of the r-th chosen expert (the pages do not say what
 * the selection writes besides the experts; the bias is a per-expert
 * correction of the choice).  Plain selection: k passes over the row. */
void oracle_router_topk(const double *logits, const double *bias, int64_t M, int64_t N, int k,
                        int32_t *idx, double *score)
{
    for (int64_t m = 0; m < M; ++m) {
        const double *z = logits + m * N;
        for (int r = 0; r < k; ++r) {
            int64_t best = -1;
            double best_v = 0.0, best_s = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                int taken = 0;
                for (int q = 0; q < r; ++q)
                    if (idx[m * k + q] == (int32_t)j)
                        taken = 1;
                if (taken)
                    continue;
                double sj;
                oracle_router_scores(&z[j], 1, &sj);
                double vj = sj + (bias ? bias[j] : 0.0);
                if (best < 0 || vj > best_v) {  /* strict: the lower index keeps a tie */
                    best = j;
                    best_v = vj;
                    best_s = sj;
                }
            }
            idx[m * k + r] = (int32_t)best;
            score[m * k + r] = best_s;
        }
    }
}

/* Threads of the parallel loops above (the benchmark's CPU baseline times
 * the oracle on every host core and on one). */
void oracle_set_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}

int oracle_max_threads(void)
{
    return omp_get_max_threads();
}
