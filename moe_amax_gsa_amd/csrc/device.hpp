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

// E4M3 decode of a non-negative finite code (0..0x7E) to float.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  float sub = (float)m * 0.001953125f;  // m * 2^-9, exact
  float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// gfx950's converters round as the scale convention asks:
// v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds fp32 to E2M1 to nearest,
// ties to even, saturating at 6, keeping the sign (-0 -> 0x8); it packs
// its two inputs into one byte, the first in the low nibble.
// v_cvt_scalef32_pk_fp8_f32 with scale 1 rounds to E4M3 to nearest even
// (NaN above 448, so the input is clamped first).  Both were compared on
// the device with bit-level round-to-nearest-even encoders on every input
// they see here (every non-negative finite fp32; every fp32 in [0, 448]).
typedef short short2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t e4m3_encode_hw(float v) {
  const short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2_t{0, 0}, fminf(v, 448.0f),
                                                              0.0f, 1.0f, false);
  return (uint32_t)(uint16_t)r[0] & 0xFFu;
}

// Eight signed quotients v[i] / sc, each correctly rounded, as E2M1 codes
// (code i in bits 4i .. 4i+3).  sc > 0.
__device__ __forceinline__ uint32_t e2m1_codes8_hw(const float v[8], float sc) {
#pragma clang fp contract(off)
  uint32_t c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[0] / sc, v[1] / sc, 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[2] / sc, v[3] / sc, 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[4] / sc, v[5] / sc, 1.0f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, v[6] / sc, v[7] / sc, 1.0f, 3);
  return c;
}

// The same codes as e2m1_codes8_hw without eight divisions.  Each quotient
// q is formed with the hardware reciprocal: q = v * rcp(sc) lies within
// 2^-22 |v / sc| of v / sc, and so of the correctly rounded quotient.  q is
// converted twice, nudged up and down by 2^-20 of itself.  Rounding to E2M1
// is monotone in the magnitude, so where both conversions agree it is
// constant over that window, which holds the correctly rounded quotient:
// its code is the agreed one.  Where they differ a rounding boundary (a
// tie) is near, and the quotients are divided exactly.  sc > 0, normal.
__device__ __forceinline__ uint32_t e2m1_codes8(const float v[8], float sc) {
#pragma clang fp contract(off)
  const float r = __builtin_amdgcn_rcpf(sc);
  float u[8], d[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = v[i] * r;
    u[i] = fmaf(q, 0x1p-20f, q);
    d[i] = fmaf(q, -0x1p-20f, q);
  }
  uint32_t up = 0, dn = 0;
  up = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(up, u[0], u[1], 1.0f, 0);
  up = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(up, u[2], u[3], 1.0f, 1);
  up = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(up, u[4], u[5], 1.0f, 2);
  up = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(up, u[6], u[7], 1.0f, 3);
  dn = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dn, d[0], d[1], 1.0f, 0);
  dn = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dn, d[2], d[3], 1.0f, 1);
  dn = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dn, d[4], d[5], 1.0f, 2);
  dn = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dn, d[6], d[7], 1.0f, 3);
  if (up == dn) return up;
  return e2m1_codes8_hw(v, sc);
}

// e4m3_encode_hw(a / b) for a >= 0, b > 0 normal, without the division
// where it is not needed: as in e2m1_codes8, the quotient from the hardware
// reciprocal is encoded nudged up and down by 2^-20 of itself (E4M3
// rounding with saturation is monotone); the exact quotient is formed only
// where the two encodings differ.
__device__ __forceinline__ uint32_t e4m3_of_quotient(float a, float b) {
#pragma clang fp contract(off)
  const float q = a * __builtin_amdgcn_rcpf(b);
  const uint32_t up = e4m3_encode_hw(fmaf(q, 0x1p-20f, q));
  const uint32_t dn = e4m3_encode_hw(fmaf(q, -0x1p-20f, q));
  if (up == dn) return up;
  return e4m3_encode_hw(a / b);
}

// Signs only (the codes of a block whose scale rounded to 0).
__device__ __forceinline__ uint32_t e2m1_signs8(const float v[8]) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) c |= ((__float_as_uint(v[i]) >> 31) << 3) << (4 * i);
  return c;
}

// silu(g) * u = g / (1 + exp(-g)) * u in fp32 with the hardware exp2 and
// reciprocal (each within about an ulp; exp(-g) is 2^(-g log2 e), whose
// argument rounding adds |g| 2^-24 relative): h is within a few 1e-7 of
// the exact value.  It is the one expression both SwiGLU paths (the
// standalone kernel and the grouped linear's epilogue) use, so they give
// identical h.  Large |g| saturates correctly: exp(-g) -> inf gives 0
// (times the sign of g), exp(-g) -> 0 gives g * u.
// limit > 0 first caps the gate from above and clamps the up value to
// [-limit, limit] (the pages name a SwiGLU limit without its formula; this
// is the reading taken).  Clamping is exact, so both paths still agree.
__device__ __forceinline__ float swiglu1(float g, float u, float limit) {
#pragma clang fp contract(off)
  if (limit > 0.f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// ---- wave64 cross-lane steps on DPP (no LDS round trip, unlike the
// bpermute that a general shuffle compiles to).  Within each row of 16
// lanes: quad_perm [1,0,3,2] pairs lane i with i ^ 1 and [2,3,0,1] with
// i ^ 2, so two steps leave every lane with its quad's result; then
// row_half_mirror pairs lane i of each 8-lane half with 7 - i (a lane of the
// other quad) and row_mirror pairs lane i with 15 - i (a lane of the other
// half).  Four steps leave the row's result in all 16 lanes, associated as
// ((l0 . l1) . (l2 . l3)) . ((l4 . l5) . (l6 . l7)) ... like an xor
// butterfly.  row_ror:4 / row_ror:8 rotate a row by 4 / 8 lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
constexpr int DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;

__device__ __forceinline__ float row16_max_f32(float v) {
  v = fmaxf(v, dpp_f32<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f32<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f32<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp_f32<DPP_MIRROR>(v));
}
__device__ __forceinline__ float row16_sum_f32(float v) {
  v += dpp_f32<DPP_XOR1>(v);
  v += dpp_f32<DPP_XOR2>(v);
  v += dpp_f32<DPP_HALF_MIRROR>(v);
  return v + dpp_f32<DPP_MIRROR>(v);
}
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_XOR1>(v));
  v = max(v, dpp_u32<DPP_XOR2>(v));
  v = max(v, dpp_u32<DPP_HALF_MIRROR>(v));
  return max(v, dpp_u32<DPP_MIRROR>(v));
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// The whole wave's result, uniform (the four rows' results read out).
__device__ __forceinline__ float wave_max_f32(float v) {
  v = row16_max_f32(v);
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = row16_sum_f32(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                 (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                 (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
// lane ^ 1 (the other half of a 16-element block in the quantize kernels)
__device__ __forceinline__ float xor1_f32(float v) { return dpp_f32<DPP_XOR1>(v); }

}  // namespace nvfp4

namespace nvfp4 {

// ---- |x| maximum as an ordered integer (bf16: 15 bits, fp32: 31 bits).
// For non-negative finite floats the bit pattern orders like the value, so
// the integer max is the exact, order-free maximum.
// A 16-byte load that is not kept in the caches (for streams larger than
// they are).
__device__ __forceinline__ uint4 load_nt16(const uint4* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool BF16>
__device__ __forceinline__ uint32_t absbits_vec(uint4 v) {
  if (BF16) {
    uint32_t a = max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu);
    uint32_t b = max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu);
    uint32_t c = max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu);
    uint32_t d = max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu);
    return max(max(a, b), max(c, d));
  }
  return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
}

// Max of |x| bits over elements tid, tid + nthreads, ... (16-byte vectors,
// scalar tail).  x must be 16-byte aligned.
// NT: nontemporal loads, for tensors larger than the Infinity Cache.
template <bool BF16, bool NT = false>
__device__ __forceinline__ uint32_t thread_absmax(const void* __restrict__ x, int64_t numel,
                                                  int64_t tid, int64_t nthreads) {
  constexpr int EPV = BF16 ? 8 : 4;
  const uint4* __restrict__ xv = (const uint4*)x;
  const int64_t nvec = numel / EPV;
  uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
  int64_t i = tid;
  auto ld = [&](int64_t k) { return NT ? load_nt16(xv + k) : xv[k]; };
  for (; i + 3 * nthreads < nvec; i += 4 * nthreads) {
    uint4 v0 = ld(i), v1 = ld(i + nthreads), v2 = ld(i + 2 * nthreads), v3 = ld(i + 3 * nthreads);
    m0 = max(m0, absbits_vec<BF16>(v0));
    m1 = max(m1, absbits_vec<BF16>(v1));
    m2 = max(m2, absbits_vec<BF16>(v2));
    m3 = max(m3, absbits_vec<BF16>(v3));
  }
  for (; i < nvec; i += nthreads) m0 = max(m0, absbits_vec<BF16>(xv[i]));
  for (int64_t e = nvec * EPV + tid; e < numel; e += nthreads) {
    uint32_t b = BF16 ? (uint32_t)((const uint16_t*)x)[e] & 0x7FFFu
                      : ((const uint32_t*)x)[e] & 0x7FFFFFFFu;
    m1 = max(m1, b);
  }
  return max(max(m0, m1), max(m2, m3));
}

// gsa = max(amax, 1e-8) / (6 * 448).
__device__ __forceinline__ float gsa_from_amax(float amax) {
#pragma clang fp contract(off)
  if (!(amax >= 1e-8f)) amax = 1e-8f;
  return amax / 2688.0f;
}

// gsa = max(amax, 1e-8) / (6 * 448) from the maximum's bits.
template <bool BF16>
__device__ __forceinline__ float gsa_from_bits(uint32_t bits) {
  return gsa_from_amax(BF16 ? __uint_as_float(bits << 16) : __uint_as_float(bits));
}

// Load the 16 elements of block b (elements 16b .. 16b+15 of a row-major
// tensor whose row length is a multiple of 16) as floats.
template <bool BF16>
__device__ __forceinline__ void load_block16(const void* __restrict__ x, int64_t b, float v[16]) {
  if (BF16) {
    const uint4* p = (const uint4*)x + 2 * b;
    const uint4 u0 = p[0], u1 = p[1];
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const uint4* p = (const uint4*)x + 4 * b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = p[i];
      v[4 * i] = __uint_as_float(u.x);
      v[4 * i + 1] = __uint_as_float(u.y);
      v[4 * i + 2] = __uint_as_float(u.z);
      v[4 * i + 3] = __uint_as_float(u.w);
    }
  }
}

__device__ __forceinline__ float block_absmax16(const float v[16]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// Quantize one 16-element block held in registers: E4M3 scale byte and 16
// E2M1 codes packed in two words (code 2i in the low nibble of byte i).
// One IEEE fp32 operation per step, no contraction:
//   sf = E4M3(bamax / (gsa * 6)), s = dec(sf) * gsa, code = sign | E2M1(|x| / s).
__device__ __forceinline__ void quantize_vals16(const float v[16], float gsa, uint32_t& lo,
                                                uint32_t& hi, uint32_t& sf) {
#pragma clang fp contract(off)
  const float bamax = block_absmax16(v);
  const float six_gsa = gsa * 6.0f;
  sf = e4m3_of_quotient(bamax, six_gsa);
  const float sdec = e4m3_decode(sf);
  const float sc = sdec * gsa;
  if (sdec == 0.0f) {  // every magnitude rounds to 0; signs stay
    lo = e2m1_signs8(v);
    hi = e2m1_signs8(v + 8);
    return;
  }
  lo = e2m1_codes8(v, sc);
  hi = e2m1_codes8(v + 8, sc);
}

// Half-block layout: thread h owns elements 8h .. 8h+7 (one 16-byte bf16
// load); half-blocks 2b and 2b+1 form block b and sit in adjacent lanes.
template <bool BF16>
__device__ __forceinline__ void load_half8(const void* __restrict__ x, int64_t h, float v[8]) {
  if (BF16) {
    const uint4 u = ((const uint4*)x)[h];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const uint4* p = (const uint4*)x + 2 * h;
    const uint4 a = p[0], b = p[1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

// The same split in two steps: raw 16-byte words first (bf16: one word,
// fp32: two), floats later -- so that a kernel can issue other loads
// before it waits for these.
template <bool BF16>
__device__ __forceinline__ void load_half8_raw(const void* __restrict__ x, int64_t h, uint4 r[2]) {
  if (BF16) {
    r[0] = ((const uint4*)x)[h];
    r[1] = make_uint4(0u, 0u, 0u, 0u);
  } else {
    const uint4* p = (const uint4*)x + 2 * h;
    r[0] = p[0];
    r[1] = p[1];
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack_half8(const uint4 r[2], float v[8]) {
  if (BF16) {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    v[0] = __uint_as_float(r[0].x); v[1] = __uint_as_float(r[0].y);
    v[2] = __uint_as_float(r[0].z); v[3] = __uint_as_float(r[0].w);
    v[4] = __uint_as_float(r[1].x); v[5] = __uint_as_float(r[1].y);
    v[6] = __uint_as_float(r[1].z); v[7] = __uint_as_float(r[1].w);
  }
}

__device__ __forceinline__ float half_absmax8(const float v[8]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// Codes of one half-block given its block's maximum: the same steps as
// quantize_vals16 (both lanes of a block compute the same scale).
__device__ __forceinline__ void quantize_half8(const float v[8], float bamax, float gsa,
                                               uint32_t& codes, uint32_t& sf) {
#pragma clang fp contract(off)
  const float six_gsa = gsa * 6.0f;
  sf = e4m3_of_quotient(bamax, six_gsa);
  const float sdec = e4m3_decode(sf);
  const float sc = sdec * gsa;
  codes = sdec == 0.0f ? e2m1_signs8(v) : e2m1_codes8(v, sc);
}

// Largest |v| of a half-block as the bits of a non-negative float (for such
// floats the integer order is the value order, so no NaN-quieting max).
__device__ __forceinline__ uint32_t half_absmax8_bits(const float v[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  return m;
}

// quantize_half8 for H half-blocks of one thread at once, with the same
// results: the reciprocal-based fast paths of all H scales, then of all H
// code words, each followed by ONE branch into the exact division for the
// (rare) lanes near a rounding tie -- so the H independent chains
// interleave instead of being cut apart by a branch per half-block.  The
// E4M3 scale decodes on gfx950's fp8 converter (OCP E4M3FN, exact).
// bamax[h]: the maximum of half-block h's whole block.
template <int H>
__device__ __forceinline__ void quantize_halves(const float (&v)[H][8], const float (&bamax)[H],
                                                float gsa, uint32_t (&codes)[H],
                                                uint32_t (&sf)[H]) {
#pragma clang fp contract(off)
  const float six_gsa = gsa * 6.0f;
  const float r6 = __builtin_amdgcn_rcpf(six_gsa);
  uint32_t dn[H];
  bool near = false;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const float q = bamax[h] * r6;
    sf[h] = e4m3_encode_hw(fmaf(q, 0x1p-20f, q));
    dn[h] = e4m3_encode_hw(fmaf(q, -0x1p-20f, q));
    near |= sf[h] != dn[h];
  }
  if (near) {
#pragma unroll
    for (int h = 0; h < H; ++h)
      if (sf[h] != dn[h]) sf[h] = e4m3_encode_hw(bamax[h] / six_gsa);
  }
  float sc[H];
  bool zero[H];
  uint32_t up8[H], dn8[H];
  near = false;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const float sdec = __builtin_amdgcn_cvt_f32_fp8((int)sf[h], 0);
    zero[h] = sdec == 0.0f;
    sc[h] = zero[h] ? 1.0f : sdec * gsa;  // a zero scale keeps signs only (below)
    const float r = __builtin_amdgcn_rcpf(sc[h]);
    float u[8], d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = v[h][i] * r;
      u[i] = fmaf(q, 0x1p-20f, q);
      d[i] = fmaf(q, -0x1p-20f, q);
    }
    uint32_t a = 0, b = 0;
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, u[0], u[1], 1.0f, 0);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, u[2], u[3], 1.0f, 1);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, u[4], u[5], 1.0f, 2);
    a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, u[6], u[7], 1.0f, 3);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, d[0], d[1], 1.0f, 0);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, d[2], d[3], 1.0f, 1);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, d[4], d[5], 1.0f, 2);
    b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, d[6], d[7], 1.0f, 3);
    up8[h] = a;
    dn8[h] = b;
    near |= !zero[h] && a != b;
  }
  if (near) {
#pragma unroll
    for (int h = 0; h < H; ++h)
      if (!zero[h] && up8[h] != dn8[h]) up8[h] = e2m1_codes8_hw(v[h], sc[h]);
  }
#pragma unroll
  for (int h = 0; h < H; ++h) codes[h] = zero[h] ? e2m1_signs8(v[h]) : up8[h];
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations (lgkmcnt 0) but leaves vector-memory loads in flight, unlike
// __syncthreads(), whose release fence also drains them.
// 16 bytes per lane from base + voff straight into LDS at byte address
// lds_wave_base + 16 * lane (base and lds_wave_base uniform over the wave).
// Issued as inline assembly so that the compiler does not fence every later
// LDS read behind it (it cannot tell the stages apart); the kernel waits
// for these loads itself with explicit vmcnt counts.  M0 carries the LDS
// address; the compiler reserves M0, so its value is saved and restored
// here, and one wait state separates the M0 write from the load.
__device__ __forceinline__ void load_lds16(const uint8_t* base, uint32_t voff,
                                           uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_wave_base), "v"(voff), "s"(base)
      : "memory");
}

// The same load, nontemporal: for data read once (an expert's weight stream),
// which should not displace what the caches hold.
__device__ __forceinline__ void load_lds16_nt(const uint8_t* base, uint32_t voff,
                                              uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_wave_base), "v"(voff), "s"(base)
      : "memory");
}

// N direct loads from one base in a single block: 16 bytes per lane from
// base + voff[i] into LDS at m0_first + i * stride + 16 * lane.  Every offset
// sits in its own register while the loads issue; computing them one at a
// time into one register would make each address wait until the previous
// load has read it.
template <int N>
__device__ __forceinline__ void load_lds16_run(const uint8_t* base, const uint32_t (&voff)[N],
                                               uint32_t m0_first, uint32_t stride) {
  static_assert(N >= 1 && N <= 8, "1 to 8 loads");
  uint32_t saved;
  if constexpr (N == 1)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %4\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "s"(base)
        : "memory");
  else if constexpr (N == 2)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %5\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %5\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "v"(voff[1]), "s"(base)
        : "memory");
  else if constexpr (N == 3)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %6\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %6\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %6\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "s"(base)
        : "memory");
  else if constexpr (N == 4)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %7\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %7\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %7\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %6, %7\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(base)
        : "memory");
  else if constexpr (N == 5)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %8\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %8\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %8\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %6, %8\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %7, %8\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "s"(base)
        : "memory");
  else if constexpr (N == 6)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %9\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %9\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %9\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %6, %9\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %7, %9\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %8, %9\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]), "s"(base)
        : "memory");
  else if constexpr (N == 7)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %10\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %10\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %10\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %6, %10\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %7, %10\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %8, %10\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %9, %10\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]), "v"(voff[6]), "s"(base)
        : "memory");
  else if constexpr (N == 8)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %11\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %11\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %11\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %6, %11\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %7, %11\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %8, %11\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %9, %11\n\t"
        "s_add_u32 m0, m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %10, %11\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0_first), "s"(stride), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]), "v"(voff[6]), "v"(voff[7]), "s"(base)
        : "memory");
}

// LDS byte address of a pointer into dynamic shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace nvfp4
