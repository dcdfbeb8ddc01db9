// device.hpp -- gfx950 device helpers shared by the NVFP4 kernels.
//
// Formats (pages of the nvfp4-megamoe-kernel repository):
//   E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
//     magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} (commit 0d1cd1e,
//     dsv4/kernels/indexer, commit message on the E2M1 decode fix).
//   E4M3 block scale: OCP FP8 E4M3FN, largest finite 448 (CORRECTNESS_BACKLOG.md,
//     section 7 "NVFP4 Quantization").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(16))) float float16_t;
typedef __attribute__((ext_vector_type(8))) int int8_t_vec;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// E4M3 encode of v >= 0: round to nearest even on the E4M3 grid, values
// above 448 saturate to 448 (0x7E).  Below 2^-6 the grid is uniform with
// step 2^-9, so the code is rint(v * 512); above it the fp32 mantissa is
// rounded to 3 bits at bit 20 and the exponent rebased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  v = fminf(v, 448.0f);
  if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (u >> 20) - ((127u - 7u) << 3);
}

// E4M3 decode of a non-negative finite code (0..0x7E) to float.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  float sub = (float)m * 0.001953125f;  // m * 2^-9, exact
  float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// E2M1 magnitude index of q >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to
// the even mantissa bit, beyond 6 -> 6.  Each comparison is one grid
// midpoint; the strict/non-strict choice at a midpoint sends the tie to the
// neighbour whose mantissa bit is 0.
__device__ __forceinline__ uint32_t e2m1_magnitude(float q) {
  return (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) +
         (uint32_t)(q >= 1.75f) + (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) +
         (uint32_t)(q > 5.0f);
}

// ---- wave64 reductions (DPP-friendly xor shuffles)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

}  // namespace nvfp4
