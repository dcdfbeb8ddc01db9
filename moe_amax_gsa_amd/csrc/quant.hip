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

// Phase 1: one partial maximum per workgroup.
template <bool BF16>
__global__ __launch_bounds__(AMAX_THREADS) void amax_partial_kernel(
    const void* __restrict__ x, int64_t numel, uint32_t* __restrict__ partials) {
  const int64_t nthreads = (int64_t)gridDim.x * AMAX_THREADS;
  uint32_t m = thread_absmax<BF16>(x, numel, (int64_t)blockIdx.x * AMAX_THREADS + threadIdx.x,
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
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += AMAX_THREADS) m = max(m, partials[i]);
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
  if (bf16) {
    amax_partial_kernel<true><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    amax_finalize_kernel<true><<<1, AMAX_THREADS, 0, s>>>(partials, parts, gsa);
  } else {
    amax_partial_kernel<false><<<parts, AMAX_THREADS, 0, s>>>(x, numel, partials);
    amax_finalize_kernel<false><<<1, AMAX_THREADS, 0, s>>>(partials, parts, gsa);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- quantize
// One thread per 16-element block.  Row-major (M, K) with K % 16 == 0 makes
// block b of the flattened tensor start at element 16b, its codes at byte 8b
// and its scale at byte b.
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, int64_t nblk,
                                                       const float* __restrict__ gsa_p,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  uint32_t lo, hi, sf;
  quantize_block16<BF16>(x, b, gsa_p[0], lo, hi, sf);
  ((uint2*)codes)[b] = make_uint2(lo, hi);
  scales[b] = (uint8_t)sf;
}

hipError_t launch_quantize(const void* x, bool bf16, int64_t M, int64_t K, const float* gsa,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblk = M * (K / 16);
  if (nblk == 0) return hipSuccess;
  const int64_t grid = (nblk + 255) / 256;
  if (bf16)
    quantize_kernel<true><<<(unsigned)grid, 256, 0, s>>>(x, nblk, gsa, codes, scales);
  else
    quantize_kernel<false><<<(unsigned)grid, 256, 0, s>>>(x, nblk, gsa, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------- SwiGLU
// Thread t handles output column c of row m; gate group 2p and up group 2p+1.
__global__ __launch_bounds__(256) void swiglu_deinterleave_kernel(const float* __restrict__ l1,
                                                                  float* __restrict__ h,
                                                                  int64_t M, int64_t NI,
                                                                  int gran) {
  const int64_t H = NI / 2;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M * H) return;
  const int64_t m = t / H, c = t - m * H;
  const int64_t pair = c / gran, off = c - pair * gran;
  const float g = l1[m * NI + 2 * pair * gran + off];
  const float u = l1[m * NI + (2 * pair + 1) * gran + off];
  h[t] = g / (1.0f + expf(-g)) * u;
}

hipError_t launch_swiglu_deinterleave(const float* l1, float* h, int64_t M, int64_t NI, int gran,
                                      hipStream_t s) {
  const int64_t n = M * (NI / 2);
  if (n == 0) return hipSuccess;
  swiglu_deinterleave_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(l1, h, M, NI, gran);
  return hipGetLastError();
}

}  // namespace nvfp4
