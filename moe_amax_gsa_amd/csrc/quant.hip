// quant.hip -- amax -> gsa (two-phase grid reduction), quantize from a gsa
// buffer, and the unfused SwiGLU de-interleave, for gfx950.
//
// Compiled with -ffp-contract=off and correctly rounded fp32 division: the
// codes and scales are bit-exact functions of the input, so every float
// operation here is one IEEE operation in the written order.
//
// Sources (nvfp4-megamoe-kernel pages):
//   gsa = max|x| / (6 * 448)        commit 107d62d, single_shot_inference.py,
//                                    commit message on the runtime gsa fix
//   amax clamp(min=1e-8), on device  deleted PERFORMANCE_AUDIT.md, section P0
//   amax kernel, then quantize that  commit 107d62d, dsv4/ops/quantize.py,
//   reads gsa from a GPU buffer      commit message (the single-pass kernel's
//                                    block barrier did not order other blocks)
//   gate/up interleave, granularity 8 README.md, MoE kernel section
#include "device.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace nvfp4 {

constexpr int AMAX_THREADS = 256;
constexpr int SMALL_THREADS = 1024;
// Tensors of at least 256 MiB outgrow the Infinity Cache: the quantize pass
// reads them from HBM again whatever the amax pass does.  For them the amax
// loads are nontemporal, and a quantize thread takes four half-blocks (more
// bytes in flight); smaller tensors stay cached between the two passes,
// where plain loads and one half-block a thread are faster (measured at
// 1.85 GB and at 29 MB).
constexpr int64_t STREAM_BYTES = 256ll << 20;
constexpr int64_t QUANTIZE_WIDE_HALVES = 1ll << 24;  // 256 MiB of bf16
// From 2^20 half-blocks (16 MiB of bf16) the amax partials take their own
// finalize launch and the quantize reads gsa; below, every quantize
// workgroup reduces the partials itself, one launch fewer.  Measured on
// MI355X, amax + quantize of (M, 7168) bf16, partials reduced in the
// quantize against a finalize launch: M = 512 8.5 against 9.5 us, 1024
// 12.0 / 12.3, 1536 13.9 / 13.7, 2048 18.6 / 17.8, 3072 26.8 / 24.5 (four
// half-blocks a thread in the quantize), 8192 50.6 / 50.6.
constexpr int64_t QUANTIZE_INLINE_MAX_HALVES = 1ll << 20;
// at most this many amax partials are reduced inside every quantize workgroup
constexpr int QUANTIZE_INLINE_PARTS = 512;

// Block-wide max; every thread gets the result.
template <int THREADS>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[THREADS / 64];
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) r = max(r, red[w]);
  return r;
}

// Phase 1: one partial maximum per workgroup.  NT: nontemporal loads (a
// tensor the caches cannot keep for the quantize pass anyway).
template <bool BF16, bool NT = false>
__global__ __launch_bounds__(AMAX_THREADS) void amax_partial_kernel(
    const void* __restrict__ x, int64_t numel, uint32_t* __restrict__ partials) {
  const int64_t nthreads = (int64_t)gridDim.x * AMAX_THREADS;
  uint32_t m = thread_absmax<BF16, NT>(x, numel, (int64_t)blockIdx.x * AMAX_THREADS + threadIdx.x,
                                       nthreads);
  m = block_max_u32<AMAX_THREADS>(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Phase 2: one workgroup reduces the partials and writes gsa.  It starts
// only after phase 1 has completed (stream order), which is the grid-wide
// barrier a block-local barrier cannot provide.
template <bool BF16>
__global__ __launch_bounds__(AMAX_THREADS) void amax_finalize_kernel(
    const uint32_t* __restrict__ partials, int nparts, float* __restrict__ gsa) {
  // eight independent loads in flight per thread, not one after another
  uint32_t m = 0;
  for (int i0 = threadIdx.x; i0 < nparts; i0 += 8 * AMAX_THREADS) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * AMAX_THREADS;
      v[u] = i < nparts ? partials[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) m = max(m, v[u]);
  }
  m = block_max_u32<AMAX_THREADS>(m);
  if (threadIdx.x == 0) gsa[0] = gsa_from_bits<BF16>(m);
}

// Small inputs: one workgroup covers the whole tensor, so the block barrier
// is a complete reduction.
template <bool BF16>
__global__ __launch_bounds__(SMALL_THREADS) void amax_single_block_kernel(
    const void* __restrict__ x, int64_t numel, float* __restrict__ gsa) {
  uint32_t m = thread_absmax<BF16>(x, numel, threadIdx.x, SMALL_THREADS);
  m = block_max_u32<SMALL_THREADS>(m);
  if (threadIdx.x == 0) gsa[0] = gsa_from_bits<BF16>(m);
}

int amax_parts_for(int64_t numel) {
  // ~16 KB of input per workgroup, at most AMAX_MAX_PARTS workgroups.
  int64_t p = (numel + 8191) / 8192;
  if (p < 1) p = 1;
  if (p > AMAX_MAX_PARTS) p = AMAX_MAX_PARTS;
  return (int)p;
}

hipError_t launch_amax_partials(const void* x, bool bf16, int64_t numel, uint32_t* partials,
                                int64_t* nparts, hipStream_t s) {
  const int parts = amax_parts_for(numel);
  *nparts = parts;
  const bool nt = numel * (bf16 ? 2 : 4) >= STREAM_BYTES;
  if (bf16) {
    if (nt)
      amax_partial_kernel<true, true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    else
      amax_partial_kernel<true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
  } else {
    if (nt)
      amax_partial_kernel<false, true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    else
      amax_partial_kernel<false><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
  }
  return hipGetLastError();
}

hipError_t launch_amax_gsa(const void* x, bool bf16, int64_t numel, float* gsa, void* ws,
                           hipStream_t s) {
  if (numel <= AMAX_SMALL_NUMEL) {
    if (bf16)
      amax_single_block_kernel<true><<<1, SMALL_THREADS, 0, s>>>(x, numel, gsa);
    else
      amax_single_block_kernel<false><<<1, SMALL_THREADS, 0, s>>>(x, numel, gsa);
    return hipGetLastError();
  }
  const int parts = amax_parts_for(numel);
  uint32_t* partials = (uint32_t*)ws;
  const bool nt = numel * (bf16 ? 2 : 4) >= STREAM_BYTES;
  if (bf16) {
    if (nt)
      amax_partial_kernel<true, true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    else
      amax_partial_kernel<true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    amax_finalize_kernel<true><<<1, AMAX_THREADS, 0, s>>>(partials, parts, gsa);
  } else {
    if (nt)
      amax_partial_kernel<false, true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    else
      amax_partial_kernel<false><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    amax_finalize_kernel<false><<<1, AMAX_THREADS, 0, s>>>(partials, parts, gsa);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- quantize
// One thread per half-block (8 elements: one 16-byte bf16 load, so a wave
// reads 1 KB contiguous); the two halves of a block are adjacent lanes and
// exchange their maxima with one shuffle.  Row-major (M, K) with K % 16 == 0
// makes half-block h start at element 8h, its 4 code bytes at byte 4h and
// its block's scale at byte h/2.
// FINALIZE: gsa is not read but formed -- every workgroup reduces the
// nparts amax partials itself (the second amax phase; the partials hold
// the bits of non-negative maxima in the input's own format: bf16 bits for
// a bf16 input, fp32 bits otherwise), and workgroup 0 writes it to
// gsa_p[0].
// HPT > 1: a workgroup covers 256 HPT half-blocks, thread t the half-blocks
// t + 256 u, every load issued before the first quantize (more bytes in
// flight per CU for large tensors).
template <bool BF16, bool FINALIZE = false, int HPT = 1>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, int64_t nhalf,
                                                       float* __restrict__ gsa_p,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       const uint32_t* __restrict__ partials,
                                                       int nparts) {
  const int64_t h0 = (int64_t)blockIdx.x * 256 * HPT + threadIdx.x;
  float v[HPT][8];
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    const int64_t h = h0 + 256 * u;
    load_half8<BF16>(x, h < nhalf ? h : 0, v[u]);
  }
  float gsa;
  if (FINALIZE) {
    uint32_t mb = 0;
    for (int i = threadIdx.x; i < nparts; i += 256) mb = max(mb, partials[i]);
    gsa = gsa_from_bits<BF16>(block_max_u32<256>(mb));
    if (blockIdx.x == 0 && threadIdx.x == 0) gsa_p[0] = gsa;
  } else {
    gsa = gsa_p[0];
  }
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    const int64_t h = h0 + 256 * u;
    const bool ok = h < nhalf;  // nhalf is even, so both lanes of a block agree
    float m = half_absmax8(v[u]);
    m = fmaxf(m, xor1_f32(m));
    uint32_t c, sf;
    quantize_half8(v[u], m, gsa, c, sf);
    if (ok) {
      ((uint32_t*)codes)[h] = c;
      if ((h & 1) == 0) scales[h >> 1] = (uint8_t)sf;
    }
  }
}

hipError_t launch_quantize(const void* x, bool bf16, int64_t M, int64_t K, const float* gsa,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nhalf = M * (K / 8);
  if (nhalf == 0) return hipSuccess;
  float* g = const_cast<float*>(gsa);  // read only: FINALIZE is off
  if (nhalf >= QUANTIZE_WIDE_HALVES) {  // four half-blocks a thread
    const int64_t grid = (nhalf + 1023) / 1024;
    if (bf16)
      quantize_kernel<true, false, 4><<<(unsigned)grid, 256, 0, s>>>(x, nhalf, g, codes, scales,
                                                                      nullptr, 0);
    else
      quantize_kernel<false, false, 4><<<(unsigned)grid, 256, 0, s>>>(x, nhalf, g, codes, scales,
                                                                       nullptr, 0);
    return hipGetLastError();
  }
  const int64_t grid = (nhalf + 255) / 256;
  if (bf16)
    quantize_kernel<true><<<(unsigned)grid, 256, 0, s>>>(x, nhalf, g, codes, scales, nullptr, 0);
  else
    quantize_kernel<false><<<(unsigned)grid, 256, 0, s>>>(x, nhalf, g, codes, scales, nullptr, 0);
  return hipGetLastError();
}

// Steps 1 and 2 on a tensor past the one-workgroup size.  Below
// QUANTIZE_INLINE_MAX_HALVES half-blocks: at most QUANTIZE_INLINE_PARTS amax
// partials (each amax workgroup takes a larger slice past that size), which
// every quantize workgroup reduces itself (two launches instead of three);
// from there on the separate finalize, and from 256 MiB the wide quantize.
hipError_t launch_amax_then_quantize(const void* x, bool bf16, int64_t M, int64_t K, float* gsa,
                                     uint8_t* codes, uint8_t* scales, void* ws, hipStream_t s) {
  const int64_t numel = M * K, nhalf = M * (K / 8);
  const int parts = amax_parts_for(numel) < QUANTIZE_INLINE_PARTS ? amax_parts_for(numel)
                                                                   : QUANTIZE_INLINE_PARTS;
  if (numel <= AMAX_SMALL_NUMEL || nhalf >= QUANTIZE_INLINE_MAX_HALVES) {
    const hipError_t e = launch_amax_gsa(x, bf16, numel, gsa, ws, s);
    if (e != hipSuccess) return e;
    return launch_quantize(x, bf16, M, K, gsa, codes, scales, s);
  }
  uint32_t* partials = (uint32_t*)ws;
  const int64_t grid = (nhalf + 255) / 256;
  if (bf16) {
    amax_partial_kernel<true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    quantize_kernel<true, true><<<(unsigned)grid, 256, 0, s>>>(x, nhalf, gsa, codes, scales,
                                                               partials, parts);
  } else {
    amax_partial_kernel<false><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    quantize_kernel<false, true><<<(unsigned)grid, 256, 0, s>>>(x, nhalf, gsa, codes, scales,
                                                                partials, parts);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_finalize(const float* x, int64_t M, int64_t K,
                                    const uint32_t* partials, int64_t nparts, float* gsa,
                                    uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nhalf = M * (K / 8);
  if (nhalf == 0) return launch_amax_finalize(partials, nparts, gsa, s);
  if (nhalf >= QUANTIZE_INLINE_MAX_HALVES) {  // the finalize launch, then the quantize
    const hipError_t e = launch_amax_finalize(partials, nparts, gsa, s);
    if (e != hipSuccess) return e;
    return launch_quantize(x, false, M, K, gsa, codes, scales, s);
  }
  const int64_t grid = (nhalf + 255) / 256;
  quantize_kernel<false, true><<<(unsigned)grid, 256, 0, s>>>(x, nhalf, gsa, codes, scales,
                                                              partials, (int)nparts);
  return hipGetLastError();
}

// ---------------------------------------------------------------- small
// amax -> gsa -> quantize of a small tensor by ONE workgroup: the block
// barrier then spans every element, so the maximum is complete before any
// block is quantized.  Each thread holds HPT half-blocks in registers
// between the two phases.
template <bool BF16, int HPT>
__global__ __launch_bounds__(SMALL_THREADS) void amax_quantize_small_kernel(
    const void* __restrict__ x, int64_t nhalf, float* __restrict__ gsa_out,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ float red[SMALL_THREADS / 64];
  float v[HPT][8];
  bool ok[HPT];
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < HPT; ++q) {
    const int64_t h = threadIdx.x + (int64_t)q * SMALL_THREADS;
    ok[q] = h < nhalf;
    load_half8<BF16>(x, ok[q] ? h : 0, v[q]);
  }
#pragma unroll
  for (int q = 0; q < HPT; ++q)
    if (ok[q]) m = fmaxf(m, half_absmax8(v[q]));
  m = wave_max_f32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float mm = 0.f;
#pragma unroll
  for (int w = 0; w < SMALL_THREADS / 64; ++w) mm = fmaxf(mm, red[w]);
  const float gsa = gsa_from_amax(mm);
  if (threadIdx.x == 0) gsa_out[0] = gsa;
#pragma unroll
  for (int q = 0; q < HPT; ++q) {
    const int64_t h = threadIdx.x + (int64_t)q * SMALL_THREADS;
    float bm = ok[q] ? half_absmax8(v[q]) : 0.f;
    bm = fmaxf(bm, xor1_f32(bm));
    uint32_t c, sf;
    quantize_half8(v[q], bm, gsa, c, sf);
    if (ok[q]) {
      ((uint32_t*)codes)[h] = c;
      if ((h & 1) == 0) scales[h >> 1] = (uint8_t)sf;
    }
  }
}

// Up to two half-blocks a thread.  With more, one workgroup's loads came out
// slower than an amax launch followed by a quantize launch (8 x 7168 bf16:
// 12.3 against 8.3 us; 6 x 7168: 11.3 against 7.2; 3 x 7168 with three
// half-blocks a thread: 7.2 against 6.7).
bool amax_quantize_small_ok(int64_t M, int64_t K) {
  return M * (K / 8) <= 2 * SMALL_THREADS;
}

template <bool BF16>
static hipError_t launch_small_t(const void* x, int64_t nhalf, float* gsa, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s) {
  if (nhalf <= SMALL_THREADS)
    amax_quantize_small_kernel<BF16, 1><<<1, SMALL_THREADS, 0, s>>>(x, nhalf, gsa, codes, scales);
  else if (nhalf <= 2 * SMALL_THREADS)
    amax_quantize_small_kernel<BF16, 2><<<1, SMALL_THREADS, 0, s>>>(x, nhalf, gsa, codes, scales);
  else
    return hipErrorInvalidValue;  // past amax_quantize_small_ok
  return hipGetLastError();
}

hipError_t launch_amax_quantize_small(const void* x, bool bf16, int64_t M, int64_t K, float* gsa,
                                      uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nhalf = M * (K / 8);
  return bf16 ? launch_small_t<true>(x, nhalf, gsa, codes, scales, s)
              : launch_small_t<false>(x, nhalf, gsa, codes, scales, s);
}

// ---------------------------------------------------------------- RMSNorm
// RMSNorm fused into the quantize, in two kernels.  y = (x * r) * w in fp32
// (two roundings, in that order), r = 1 / sqrt(sum(x^2) / K + eps) per row.
// Kernel 1, one workgroup per row: the sum of squares, r, then the largest
// |y| of the row (y is formed as kernel 2 forms it, so the maximum is of
// the values that are quantized).  Per-row scales: it writes gsa[m]
// directly.  One scale: it writes the row maximum as a partial, a single
// workgroup reduces the partials into gsa (the grid-wide phase), and
// kernel 2 reads gsa[0].  Kernel 2 forms y again per half-block and
// quantizes it as quantize_kernel does.
__device__ __forceinline__ float block_sum_f32(float v, float* red) {
  v = wave_sum_f32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  __syncthreads();
  return t;
}

template <bool XBF16, bool WBF16>
__device__ __forceinline__ void rms_y8(const void* x, const void* w, int64_t hx, int64_t hw,
                                       float r, float y[8]) {
#pragma clang fp contract(off)
  float xv[8], wv[8];
  load_half8<XBF16>(x, hx, xv);
  load_half8<WBF16>(w, hw, wv);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (xv[i] * r) * wv[i];
}

template <bool XBF16, bool WBF16, bool PER_ROW>
__global__ __launch_bounds__(256) void rmsnorm_stats_kernel(
    const void* __restrict__ x, const void* __restrict__ w, float eps, int64_t K,
    float* __restrict__ inv_rms, float* __restrict__ gsa, uint32_t* __restrict__ partials) {
#pragma clang fp contract(off)
  __shared__ float red[4];
  const int64_t m = blockIdx.x, K8 = K / 8;
  float ss = 0.f;
  for (int64_t h = threadIdx.x; h < K8; h += 256) {
    float v[8];
    load_half8<XBF16>(x, m * K8 + h, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  }
  ss = block_sum_f32(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)K + eps);
  float mx = 0.f;
  for (int64_t h = threadIdx.x; h < K8; h += 256) {
    float y[8];
    rms_y8<XBF16, WBF16>(x, w, m * K8 + h, h, r, y);
    mx = fmaxf(mx, half_absmax8(y));
  }
  const uint32_t mb = block_max_u32<256>(__float_as_uint(mx));
  if (threadIdx.x == 0) {
    inv_rms[m] = r;
    if (PER_ROW)
      gsa[m] = gsa_from_amax(__uint_as_float(mb));
    else
      partials[m] = mb;
  }
}

// FINALIZE (one scale over several rows): every workgroup first reduces the
// nparts row maxima itself -- the second amax phase -- and workgroup 0
// writes gsa[0]; otherwise gsa is read (per row, or the finalized one).
template <bool XBF16, bool WBF16, bool PER_ROW, bool FINALIZE>
__global__ __launch_bounds__(256) void rmsnorm_quantize_kernel(
    const void* __restrict__ x, const void* __restrict__ w, int64_t K, int64_t nhalf,
    const float* __restrict__ inv_rms, float* __restrict__ gsa_p,
    const uint32_t* __restrict__ partials, int nparts, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = h < nhalf;  // nhalf is even, so both lanes of a block agree
  const int64_t K8 = K / 8, hh = ok ? h : 0, m = hh / K8;
  float y[8];
  rms_y8<XBF16, WBF16>(x, w, hh, hh - m * K8, inv_rms[m], y);
  float gsa;
  if (FINALIZE) {
    uint32_t mb = 0;
    for (int i = threadIdx.x; i < nparts; i += 256) mb = max(mb, partials[i]);
    gsa = gsa_from_amax(__uint_as_float(block_max_u32<256>(mb)));
    if (blockIdx.x == 0 && threadIdx.x == 0) gsa_p[0] = gsa;
  } else {
    gsa = gsa_p[PER_ROW ? m : 0];
  }
  float bm = half_absmax8(y);
  bm = fmaxf(bm, xor1_f32(bm));
  uint32_t c, sf;
  quantize_half8(y, bm, gsa, c, sf);
  if (ok) {
    ((uint32_t*)codes)[h] = c;
    if ((h & 1) == 0) scales[h >> 1] = (uint8_t)sf;
  }
}

constexpr int64_t RMS_INLINE_ROWS = 4096;

// One row per workgroup, the whole row in registers: thread t owns
// half-blocks t, t + T, ... (HPT of them) of the row.  The sum of squares,
// inv_rms, y = (x * inv_rms) * w, the row's largest |y| -- its gsa, the
// row's own (per-row scales, or one row) -- and the codes and scales, all
// from one read of x and w.  The two reductions over the row go through DPP
// within waves and LDS across them, each followed by one barrier.
template <bool XBF16, bool WBF16, int HPT>
__global__ __launch_bounds__(1024) void rmsnorm_quantize_row_kernel(
    const void* __restrict__ x, const void* __restrict__ w, float eps, int K,
    float* __restrict__ inv_rms, float* __restrict__ gsa_p, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
#pragma clang fp contract(off)
  __shared__ float red_s[16], red_m[16];
  const int64_t m = blockIdx.x;
  const int T = blockDim.x, nw = T >> 6, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nh = K / 8;  // half-blocks in the row
  float v[HPT][8];
  bool ok[HPT];
  uint4 xr[HPT][2], wr[HPT][2];
#pragma unroll
  for (int u = 0; u < HPT; ++u) {  // every load first
    const int h = threadIdx.x + u * T;
    ok[u] = h < nh;
    const int hc = ok[u] ? h : 0;
    load_half8_raw<XBF16>(x, m * nh + hc, xr[u]);
    load_half8_raw<WBF16>(w, hc, wr[u]);
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    unpack_half8<XBF16>(xr[u], v[u]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!ok[u]) v[u][i] = 0.f;
      ss += v[u][i] * v[u][i];
    }
  }
  ss = wave_sum_f32(ss);
  if (lane == 0) red_s[wave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < nw; ++i) tot += red_s[i];
  const float r = 1.0f / sqrtf(tot / (float)K + eps);
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    float wv[8];
    unpack_half8<WBF16>(wr[u], wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[u][i] = (v[u][i] * r) * wv[i];
    mx = fmaxf(mx, half_absmax8(v[u]));  // masked half-blocks are 0
  }
  mx = wave_max_f32(mx);
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  float rm = 0.f;
  for (int i = 0; i < nw; ++i) rm = fmaxf(rm, red_m[i]);
  const float gsa = gsa_from_amax(rm);
  if (threadIdx.x == 0) {
    inv_rms[m] = r;
    gsa_p[m] = gsa;
  }
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    const int h = threadIdx.x + u * T;
    float bm = half_absmax8(v[u]);
    bm = fmaxf(bm, xor1_f32(bm));  // T is a multiple of 64: h ^ 1 is the next lane
    uint32_t c, sf;
    quantize_half8(v[u], bm, gsa, c, sf);
    if (ok[u]) {
      ((uint32_t*)codes)[m * nh + h] = c;
      if ((h & 1) == 0) scales[m * nh / 2 + h / 2] = (uint8_t)sf;
    }
  }
}

// Threads and half-blocks per thread of the one-row kernel, or false when a
// row is too long for registers (more than 4096 half-blocks: K > 32768).
static bool rms_row_plan(int64_t K, int& threads, int& hpt) {
  const int64_t nh = K / 8;
  if (nh > 4096) return false;
  hpt = nh <= 1024 ? 1 : nh <= 2048 ? 2 : 4;
  const int64_t t = (nh + hpt - 1) / hpt;
  threads = (int)(((t + 63) / 64) * 64);
  return true;
}

template <bool XBF16, bool WBF16>
static hipError_t launch_rms_row_t(const void* x, const void* w, float eps, int64_t M, int64_t K,
                                   float* gsa, float* inv_rms, uint8_t* codes, uint8_t* scales,
                                   int threads, int hpt, hipStream_t s) {
#define RMS_ROW(H)                                                                       \
  rmsnorm_quantize_row_kernel<XBF16, WBF16, H><<<(unsigned)M, threads, 0, s>>>(x, w, eps, (int)K, \
                                                                       inv_rms, gsa, codes, \
                                                                       scales)
  if (hpt == 1)
    RMS_ROW(1);
  else if (hpt == 2)
    RMS_ROW(2);
  else
    RMS_ROW(4);
#undef RMS_ROW
  return hipGetLastError();
}

template <bool XBF16, bool WBF16, bool PER_ROW>
static hipError_t launch_rmsnorm_t(const void* x, const void* w, float eps, int64_t M, int64_t K,
                                   float* gsa, float* inv_rms, uint8_t* codes, uint8_t* scales,
                                   uint32_t* partials, hipStream_t s) {
  // per-row scales, or a single row: every scale is one row's own -- one kernel
  int threads = 0, hpt = 0;
  if ((PER_ROW || M == 1) && rms_row_plan(K, threads, hpt))
    return launch_rms_row_t<XBF16, WBF16>(x, w, eps, M, K, gsa, inv_rms, codes, scales, threads,
                                          hpt, s);
  rmsnorm_stats_kernel<XBF16, WBF16, PER_ROW><<<(unsigned)M, 256, 0, s>>>(x, w, eps, K, inv_rms,
                                                                         gsa, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nhalf = M * (K / 8);
  const unsigned grid = (unsigned)((nhalf + 255) / 256);
  // one scale over up to RMS_INLINE_ROWS rows: the quantize reduces the row
  // maxima itself (two kernels); more rows: a finalize kernel between
  if (!PER_ROW && M <= RMS_INLINE_ROWS) {
    rmsnorm_quantize_kernel<XBF16, WBF16, false, true><<<grid, 256, 0, s>>>(
        x, w, K, nhalf, inv_rms, gsa, partials, (int)M, codes, scales);
    return hipGetLastError();
  }
  if (!PER_ROW) {
    amax_finalize_kernel<false><<<1, AMAX_THREADS, 0, s>>>(partials, (int)M, gsa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  rmsnorm_quantize_kernel<XBF16, WBF16, PER_ROW, false><<<grid, 256, 0, s>>>(
      x, w, K, nhalf, inv_rms, gsa, partials, (int)M, codes, scales);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const void* x, bool x_bf16, const void* w, bool w_bf16,
                                   float eps, int64_t M, int64_t K, bool per_row, float* gsa,
                                   float* inv_rms, uint8_t* codes, uint8_t* scales,
                                   uint32_t* partials, hipStream_t s) {
  if (M == 0) return hipSuccess;
#define RMS_CASE(XB, WB, PR)                                                                   \
  if (x_bf16 == XB && w_bf16 == WB && per_row == PR)                                           \
    return launch_rmsnorm_t<XB, WB, PR>(x, w, eps, M, K, gsa, inv_rms, codes, scales, partials, \
                                        s);
  RMS_CASE(true, true, true) RMS_CASE(true, true, false) RMS_CASE(true, false, true)
  RMS_CASE(true, false, false) RMS_CASE(false, true, true) RMS_CASE(false, true, false)
  RMS_CASE(false, false, true) RMS_CASE(false, false, false)
#undef RMS_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- SwiGLU
// Thread t handles output column c of row m; gate group 2p and up group 2p+1.
__global__ __launch_bounds__(256) void swiglu_deinterleave_kernel(const float* __restrict__ l1,
                                                                  float* __restrict__ h,
                                                                  int64_t M, int64_t NI,
                                                                  int gran, float limit) {
  const int64_t H = NI / 2;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M * H) return;
  const int64_t m = t / H, c = t - m * H;
  const int64_t pair = c / gran, off = c - pair * gran;
  const float g = l1[m * NI + 2 * pair * gran + off];
  const float u = l1[m * NI + (2 * pair + 1) * gran + off];
  h[t] = swiglu1(g, u, limit);
}

hipError_t launch_amax_finalize(const uint32_t* partials, int64_t nparts, float* gsa,
                                hipStream_t s) {
  amax_finalize_kernel<false><<<1, AMAX_THREADS, 0, s>>>(partials, (int)nparts, gsa);
  return hipGetLastError();
}

hipError_t launch_swiglu_deinterleave(const float* l1, float* h, int64_t M, int64_t NI, int gran,
                                      float limit, hipStream_t s) {
  const int64_t n = M * (NI / 2);
  if (n == 0) return hipSuccess;
  swiglu_deinterleave_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(l1, h, M, NI, gran,
                                                                        limit);
  return hipGetLastError();
}

}  // namespace nvfp4
