// gemm.hip -- tiled NVFP4 linear for many activation rows (prefill), on
// gfx950 f16 matrix cores.
//
// y = gsa * ws2 * (A_codes*sfa) @ (W_codes*sfw)^T with FP32 accumulation:
// the matrix cores compute (A*SFA) @ (B*SFB) and the epilogue multiplies by
// gsa * gsb, gsb = weight_scale_2 (dsv4/_archive/layers/linear.py,
// finalize_weights comment; CORRECTNESS_BACKLOG.md section 7).
//
// Exact dequantization.  Every E2M1 magnitude times every E4M3 scale has at
// most 6 significant bits and lies in [2^-10, 2688], so lut[c] * sf is exact
// in f16 (and in bf16).  gfx950 converts packed E2M1 to f16 in hardware, but
// its operand scale applies only a power of two, so the E4M3 scale (3
// mantissa bits) is applied with a packed f16 multiply -- which gfx950 has
// for f16 and not for bf16.  Products of the exact f16 operands are exact in
// the FP32 accumulator, so this is the same arithmetic as a bf16 path.
//
// Operand layout of v_mfma_f32_32x32x16_f16: lane l holds row l % 32 and 8
// K-elements of K slice l / 32; result register r of lane l is row
// 8(r/4) + 4(l/32) + r%4, column l % 32.  The K order inside a 64-element
// step is permuted identically for both operands (the sum does not depend
// on it): lane half h owns elements [32h, 32h+32) of the step -- 16
// contiguous code bytes, two NVFP4 blocks -- and feeds elements
// [32h + 8s, +8) to MFMA s, so each MFMA operand register set lies in one
// block and takes one scale.
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma_f16(half8_t a, half8_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 8 codes (one dword, code 2i in the low nibble of byte i) times a scale.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t sf) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  p0 = p0 * sf;
  p1 = p1 * sf;
  p2 = p2 * sf;
  p3 = p3 * sf;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Both E4M3 scale bytes of a fragment's two blocks (low byte first) as f16.
__device__ __forceinline__ half2_t scale_pair2(uint32_t two) {
  const _Float16 f0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)two, 0);
  const _Float16 f1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)two, 1);
  return half2_t{f0, f1};
}

// Streaming 16-byte load (weights are read by few workgroups).
__device__ __forceinline__ uint4 ldg_nt16_g(const uint8_t* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ half2_t scale_pair(uint32_t byte) {
  const _Float16 f = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
  return half2_t{f, f};
}

// 16 code bytes and 2 scale bytes of one fragment row for K step ks.
template <bool FASTK>
__device__ __forceinline__ void load_frag(const uint8_t* crow, const uint8_t* srow, int64_t cbytes,
                                          int64_t sbytes, int ks, int h, uint4& c, uint32_t& s) {
  const int64_t co = (int64_t)ks * 32 + 16 * h;
  const int64_t so = (int64_t)ks * 4 + 2 * h;
  if (FASTK) {
    c = *(const uint4*)(crow + co);
    s = *(const uint16_t*)(srow + so);
  } else {
    const bool v0 = co + 8 <= cbytes, v1 = co + 16 <= cbytes;
    const uint2 q0 = v0 ? *(const uint2*)(crow + co) : make_uint2(0u, 0u);
    const uint2 q1 = v1 ? *(const uint2*)(crow + co + 8) : make_uint2(0u, 0u);
    c = make_uint4(q0.x, q0.y, q1.x, q1.y);
    const uint32_t s0 = so < sbytes ? srow[so] : 0u;
    const uint32_t s1 = so + 1 < sbytes ? srow[so + 1] : 0u;
    s = s0 | (s1 << 8);
  }
}

// Workgroup tile 128 x 128, four waves of 64 x 64 (2 x 2 MFMA tiles).
template <bool FASTK>
__global__ __launch_bounds__(256) void gemm_f16_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ gsa_p, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ ws2_p, void* __restrict__ y,
    int y_bf16, int M, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * 128 + wm * 64, n0 = blockIdx.x * 128 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t cbytes = K / 2, sbytes = K / 16;

  const uint8_t* ac[2];
  const uint8_t* as[2];
  const uint8_t* bc[2];
  const uint8_t* bs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t ra = min(m0 + i * 32 + r32, M - 1);  // clamped rows: results discarded
    const int64_t rb = min(n0 + i * 32 + r32, N - 1);
    ac[i] = a_codes + ra * cbytes;
    as[i] = a_scales + ra * sbytes;
    bc[i] = w_codes + rb * cbytes;
    bs[i] = w_scales + rb * sbytes;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nks = (K + 63) / 64;
  for (int ks = 0; ks < nks; ++ks) {
    uint4 ca[2], cb[2];
    uint32_t sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      load_frag<FASTK>(ac[i], as[i], cbytes, sbytes, ks, h, ca[i], sa[i]);
      load_frag<FASTK>(bc[i], bs[i], cbytes, sbytes, ks, h, cb[i], sb[i]);
    }
    half8_t A[2][4], B[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const half2_t fa0 = scale_pair(sa[i] & 0xFFu), fa1 = scale_pair(sa[i] >> 8);
      const half2_t fb0 = scale_pair(sb[i] & 0xFFu), fb1 = scale_pair(sb[i] >> 8);
      A[i][0] = dequant8(ca[i].x, fa0);
      A[i][1] = dequant8(ca[i].y, fa0);
      A[i][2] = dequant8(ca[i].z, fa1);
      A[i][3] = dequant8(ca[i].w, fa1);
      B[i][0] = dequant8(cb[i].x, fb0);
      B[i][1] = dequant8(cb[i].y, fb0);
      B[i][2] = dequant8(cb[i].z, fb1);
      B[i][3] = dequant8(cb[i].w, fb1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma_f16(A[a][s], B[b][s], acc[a][b]);
  }

  const float gscale = gsa_p[0] * ws2_p[0];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + a * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int col = n0 + b * 32 + r32;
        if (row < M && col < N) {
          const float v = acc[a][b][r] * gscale;
          if (y_bf16)
            ((uint16_t*)y)[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            ((float*)y)[(int64_t)row * N + col] = v;
        }
      }
}

// ---------------------------------------------------------------- split-K
// Workgroup tile (32*WM) x (32*WN), four waves that each compute the whole
// tile over every fourth 64-element K step -- each wave then dequantizes
// WM + WN fragments per WM*WN MFMAs (4 + 4 for 16 at 4 x 4), which keeps the
// exact f16 dequantization within the VALU slots beside the matrix cores --
// then an LDS reduction of the four partial tiles.  Codes and scales of the
// next K step are loaded while the current one computes (two register sets,
// the loop unrolled by two so that the sets are named, not indexed).
template <int WM, int WN>
struct FragSet {
  uint4 ca[WM], cb[WN];
  uint32_t sa[WM], sb[WN];
};

template <int WM, int WN>
__device__ __forceinline__ void load_set(FragSet<WM, WN>& f, const uint8_t* __restrict__ a_codes,
                                         const uint8_t* __restrict__ a_scales,
                                         const uint8_t* __restrict__ w_codes,
                                         const uint8_t* __restrict__ w_scales,
                                         const uint32_t (&aoff)[WM], const uint32_t (&asoff)[WM],
                                         const uint32_t (&boff)[WN], const uint32_t (&bsoff)[WN],
                                         int ks, int h) {
  const uint32_t co = (uint32_t)ks * 32 + 16 * h, so = (uint32_t)ks * 4 + 2 * h;
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    f.ca[i] = *(const uint4*)(a_codes + (aoff[i] + co));
    f.sa[i] = *(const uint16_t*)(a_scales + (asoff[i] + so));
  }
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    f.cb[i] = ldg_nt16_g(w_codes + (boff[i] + co));
    f.sb[i] = *(const uint16_t*)(w_scales + (bsoff[i] + so));
  }
}

template <int WM, int WN>
__device__ __forceinline__ void compute_set(const FragSet<WM, WN>& f, f32x16 (&acc)[WM][WN]) {
  half2_t sfa[WM], sfb[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) sfa[i] = scale_pair2(f.sa[i]);
#pragma unroll
  for (int i = 0; i < WN; ++i) sfb[i] = scale_pair2(f.sb[i]);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    half8_t A[WM], B[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const uint32_t w = s == 0 ? f.ca[i].x : s == 1 ? f.ca[i].y : s == 2 ? f.ca[i].z : f.ca[i].w;
      const _Float16 sc = s < 2 ? sfa[i][0] : sfa[i][1];
      A[i] = dequant8(w, half2_t{sc, sc});
    }
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const uint32_t w = s == 0 ? f.cb[i].x : s == 1 ? f.cb[i].y : s == 2 ? f.cb[i].z : f.cb[i].w;
      const _Float16 sc = s < 2 ? sfb[i][0] : sfb[i][1];
      B[i] = dequant8(w, half2_t{sc, sc});
    }
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
      for (int b = 0; b < WN; ++b) acc[a][b] = mfma_f16(A[a], B[b], acc[a][b]);
    // one substep's operands live at a time
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int WM, int WN, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void gemm_splitk4_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ gsa_p, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ ws2_p, void* __restrict__ y,
    int y_bf16, int M, int N, int K) {
  constexpr int TM = 32 * WM, TN = 32 * WN, LDT = TN + 4;
  extern __shared__ __attribute__((aligned(16))) float red[];  // [4 waves][16][LDT]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int64_t cbytes = K / 2, sbytes = K / 16;
  // 32-bit byte offsets of each fragment row (the host checks the sizes fit)
  uint32_t aoff[WM], asoff[WM], boff[WN], bsoff[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const uint32_t ra = (uint32_t)min(m0 + i * 32 + r32, M - 1);  // clamped: results discarded
    aoff[i] = ra * (uint32_t)cbytes;
    asoff[i] = ra * (uint32_t)sbytes;
  }
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    const uint32_t rb = (uint32_t)min(n0 + i * 32 + r32, N - 1);
    boff[i] = rb * (uint32_t)cbytes;
    bsoff[i] = rb * (uint32_t)sbytes;
  }
  f32x16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // wave w takes K steps w, w + 4, ...: `mine` of them, in pairs and then
  // an odd one, so the loop has a single exit and the accumulators stay put
  const int nks = K / 64;
  const int mine = wave < nks ? (nks - 1 - wave) / 4 + 1 : 0;
  FragSet<WM, WN> X, Yb;
  int ks = min(wave, nks - 1);
  load_set<WM, WN>(X, a_codes, a_scales, w_codes, w_scales, aoff, asoff, boff, bsoff, ks, h);
  for (int p = 0; p < mine / 2; ++p) {
    load_set<WM, WN>(Yb, a_codes, a_scales, w_codes, w_scales, aoff, asoff, boff, bsoff,
                     min(ks + 4, nks - 1), h);
    compute_set<WM, WN>(X, acc);
    load_set<WM, WN>(X, a_codes, a_scales, w_codes, w_scales, aoff, asoff, boff, bsoff,
                     min(ks + 8, nks - 1), h);
    compute_set<WM, WN>(Yb, acc);
    ks += 8;
  }
  if (mine & 1) compute_set<WM, WN>(X, acc);

  // reduce the four partial tiles one 16-row slab at a time (result
  // registers 8q..8q+7 of MFMA tile row a hold rows 32a + 16q + [0, 16))
  const float gscale = gsa_p[0] * ws2_p[0];
  float* slab = red + (size_t)wave * 16 * LDT;
#pragma unroll
  for (int a = 0; a < WM; ++a) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int b = 0; b < WN; ++b)
#pragma unroll
        for (int r = 8 * q; r < 8 * q + 8; ++r)
          slab[(8 * ((r >> 2) & 1) + 4 * h + (r & 3)) * LDT + b * 32 + r32] = acc[a][b][r];
      __syncthreads();
      // wave w sums rows [4w, 4w + 4) of the slab
      for (int e = lane; e < 4 * TN; e += 64) {
        const int rr = wave * 4 + e / TN, cc = e % TN;
        const float v = red[(0 * 16 + rr) * LDT + cc] + red[(1 * 16 + rr) * LDT + cc] +
                        red[(2 * 16 + rr) * LDT + cc] + red[(3 * 16 + rr) * LDT + cc];
        const int row = m0 + a * 32 + q * 16 + rr, col = n0 + cc;
        if (row < M && col < N) {
          const float o = v * gscale;
          if (y_bf16)
            ((uint16_t*)y)[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(o);
          else
            ((float*)y)[(int64_t)row * N + col] = o;
        }
      }
      __syncthreads();
    }
  }
}

template <int WM, int WN, int WPE>
hipError_t launch_splitk4(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                          void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  constexpr int TM = 32 * WM, TN = 32 * WN;
  const size_t lds = (size_t)4 * 16 * (TN + 4) * sizeof(float);
  const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
  gemm_splitk4_kernel<WM, WN, WPE><<<grid, 256, lds, s>>>(a_codes, a_scales, gsa, w_codes,
                                                          w_scales, ws2, y, y_bf16 ? 1 : 0,
                                                          (int)M, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                       void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const bool fast = (K % 64 == 0) && (((uintptr_t)a_codes | (uintptr_t)w_codes) & 15u) == 0 &&
                    (((uintptr_t)a_scales | (uintptr_t)w_scales) & 1u) == 0;
  // split-K tiles address rows with 32-bit byte offsets
  const bool big = fast && K >= 256 && M * (K / 2) < (1ll << 31) && N * (K / 2) < (1ll << 31);
  if (big) {
    const int64_t tiles44 = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles44 >= 512)
      return launch_splitk4<4, 4, 1>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16, M,
                                     N, K, s);
    return launch_splitk4<4, 2, 2>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16, M,
                                   N, K, s);
  }
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
  if (fast)
    gemm_f16_kernel<true><<<grid, 256, 0, s>>>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y,
                                               y_bf16 ? 1 : 0, (int)M, (int)N, (int)K);
  else
    gemm_f16_kernel<false><<<grid, 256, 0, s>>>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y,
                                                y_bf16 ? 1 : 0, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace nvfp4
