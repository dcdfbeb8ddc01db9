// gemv.hip -- weight-streaming NVFP4 linear for few activation rows (decode,
// routed experts), on gfx950 FP4 matrix cores.
//
// y[m, n] = gsa * ws2 * sum_b sfa[m, b] * sfw[n, b] * S_b[m, n],
// S_b[m, n] = sum over the 16 elements k of block b of lut[a] * lut[w].
// (GEMM form: dsv4/_archive/layers/linear.py, finalize_weights comment;
// weight_scale_2 fold: commit db07d17's message; per-group ws2 with one
// shared gsa: dsv4/_archive/layers/grouped_linear.py, _run_impl.)
//
// Design.  v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands multiplies
// a 16 x 128 A tile by a 128 x 16 B tile.  B holds 16 weight rows (one per
// column) exactly as stored, so the weight stream needs no conversion at
// all.  A holds "block-masked" activation rows: row i of A carries only the
// 16 codes of one NVFP4 block and zeros elsewhere, so output row i is the
// block dot product S_b for 16 weight rows -- exact (sums of multiples of
// 1/4 below 2^10).  The hardware's power-of-two operand scales stay at 1;
// each S_b is scaled by its E4M3 pair in one FP32 FMA.  Eight blocks of one
// activation row fill A rows 0..7, a second activation row fills rows 8..15.
//
// Lane geometry of the 16x16x128 FP4 MFMA (lane l, 64 lanes): A row / B
// column l % 16, K slice l / 16 of 32 codes (16 bytes); result lane l holds
// rows 4*(l/16) .. +3 of column l % 16.  A workgroup owns 16 weight rows; its
// waves split the K dimension in 256-element super-chunks (128 bytes per row,
// two MFMAs), and a lane's 32 bytes of a super-chunk are K slice j of MFMA 0
// (first 16 bytes) and MFMA 1 (next 16).  Slice j of MFMA h spans blocks
// 16c + 4j + 2h and +1, so A row i (slot s = i % 8) takes the half s % 2 of
// slice s / 2.  Result row i of MFMA h is block 16c + 8(j%2) + 4(r/2) + 2h +
// (r%2) for lane slice j and register r, whose two scale bytes sit in one
// 8-byte word per row at byte 16c + 8(j%2).
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef __attribute__((ext_vector_type(8))) int v8i;

__device__ __forceinline__ float4_t mfma_fp4(v8i a, v8i b) {
  const float4_t z = {0.f, 0.f, 0.f, 0.f};
  // cbsz = blgp = 4: both operands E2M1; operand scale bytes 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 0, 127, 0, 127);
}

// 32 code bytes of a row at byte offset off, zero outside [0, rowbytes) or
// when !ok.  FAST: the whole super-chunk is inside the row and 16-byte
// aligned.  Otherwise 8-byte pieces (rows are 8-byte aligned since K % 16 == 0).
template <bool FAST>
__device__ __forceinline__ void load32(const uint8_t* row, int64_t off, int64_t rowbytes, bool ok,
                                       uint4& a, uint4& b) {
  if (FAST) {
    if (ok) {
      const uint4* p = (const uint4*)(row + off);
      a = p[0];
      b = p[1];
    } else {
      a = b = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    uint2 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t o = off + 8 * i;
      q[i] = (ok && o + 8 <= rowbytes) ? *(const uint2*)(row + o) : make_uint2(0u, 0u);
    }
    a = make_uint4(q[0].x, q[0].y, q[1].x, q[1].y);
    b = make_uint4(q[2].x, q[2].y, q[3].x, q[3].y);
  }
}

// 8 scale bytes at row + off; zero outside the row or when !ok (a zero scale
// byte decodes to 0, never NaN).
template <bool FAST>
__device__ __forceinline__ uint2 load8(const uint8_t* row, int64_t off, int64_t rowbytes, bool ok) {
  if (FAST) return ok ? *(const uint2*)(row + off) : make_uint2(0u, 0u);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t o = off + i;
    const uint32_t byte = (ok && o < rowbytes) ? (uint32_t)row[o] : 0u;
    if (i < 4)
      w0 |= byte << (8 * i);
    else
      w1 |= byte << (8 * (i - 4));
  }
  return make_uint2(w0, w1);
}

__device__ __forceinline__ void fp8x8_to_f32(uint2 s, float f[8]) {
  f[0] = __builtin_amdgcn_cvt_f32_fp8((int)s.x, 0);
  f[1] = __builtin_amdgcn_cvt_f32_fp8((int)s.x, 1);
  f[2] = __builtin_amdgcn_cvt_f32_fp8((int)s.x, 2);
  f[3] = __builtin_amdgcn_cvt_f32_fp8((int)s.x, 3);
  f[4] = __builtin_amdgcn_cvt_f32_fp8((int)s.y, 0);
  f[5] = __builtin_amdgcn_cvt_f32_fp8((int)s.y, 1);
  f[6] = __builtin_amdgcn_cvt_f32_fp8((int)s.y, 2);
  f[7] = __builtin_amdgcn_cvt_f32_fp8((int)s.y, 3);
}

// MP activation-row pairs per pass (up to 2*MP rows); pairs past the last
// row of the pass are skipped.  GROUPED: blockIdx.y is the group; its rows
// come from offsets[], its activation rows from row_index[] (or identity).
template <int NW, int MP, bool FAST, bool GROUPED>
__global__ __launch_bounds__(NW * 64) void gemv_fp4_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ gsa_p, const int32_t* __restrict__ row_index,
    const int32_t* __restrict__ offsets, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ ws2_p, void* __restrict__ y,
    int y_bf16, int M, int N, int K, int a_rows) {
  constexpr int ROWS = 2 * MP;
  static_assert(NW * 64 >= ROWS * 16, "final reduction needs ROWS*16 threads");
  __shared__ float red[NW][ROWS][16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, j = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int g = GROUPED ? (int)blockIdx.y : 0;
  int r_begin = 0, r_end = M;
  if (GROUPED) {
    r_begin = max(offsets[g], 0);
    r_end = min(offsets[g + 1], M);
    if (r_begin >= r_end) return;  // uniform over the workgroup
  }
  const int64_t cbytes = K / 2, sbytes = K / 16;
  const int64_t n_here = (n0 + col < N) ? n0 + col : n0;  // clamp: results discarded
  const uint8_t* wrow = w_codes + ((int64_t)g * N + n_here) * cbytes;
  const uint8_t* wsrow = w_scales + ((int64_t)g * N + n_here) * sbytes;
  const int nsc = (K + 255) / 256;
  const float gscale = gsa_p[0] * ws2_p[g];

  // A operand: lane row i = col -> local row 2p + (i / 8), slot s = i % 8,
  // carries data only when s / 2 == j, in half s % 2.
  const int a_mloc = col >> 3, a_half = col & 1;
  const bool a_has = ((col & 7) >> 1) == j;
  // Result: lane rows 4j .. 4j+3 belong to local row 2p + j / 2.
  const int c_mloc = j >> 1;

  for (int r0 = r_begin; r0 < r_end; r0 += ROWS) {
    const uint8_t* ac[MP];
    const uint8_t* as[MP];
    bool aok[MP], sok[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) {
      const int ra = r0 + 2 * p + a_mloc;
      const int rc = r0 + 2 * p + c_mloc;
      aok[p] = a_has && ra < r_end;
      sok[p] = rc < r_end;
      int64_t rowa = ra < r_end ? ra : r0, rowc = rc < r_end ? rc : r0;
      if (GROUPED && row_index != nullptr) {
        rowa = row_index[rowa];
        rowc = row_index[rowc];
        // an index outside the activation rows reads nothing (its row is
        // not written either)
        if (rowa < 0 || rowa >= a_rows) { rowa = 0; aok[p] = false; }
        if (rowc < 0 || rowc >= a_rows) { rowc = 0; sok[p] = false; }
      }
      ac[p] = a_codes + rowa * cbytes;
      as[p] = a_scales + rowc * sbytes;
    }
    float acc[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) acc[p] = 0.f;

    for (int c = wave; c < nsc; c += NW) {
      const int64_t boff = (int64_t)c * 128 + 32 * j;
      const int64_t soff = (int64_t)c * 16 + 8 * (j & 1);
      uint4 w0, w1;
      load32<FAST>(wrow, boff, cbytes, true, w0, w1);
      const uint2 sw = load8<FAST>(wsrow, soff, sbytes, true);
      const v8i B0 = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, 0, 0, 0, 0};
      const v8i B1 = {(int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w, 0, 0, 0, 0};
      float fw[8];
      fp8x8_to_f32(sw, fw);
#pragma unroll
      for (int p = 0; p < MP; ++p) {
        if (r0 + 2 * p >= r_end) break;  // uniform
        uint4 a0, a1;
        load32<FAST>(ac[p], boff, cbytes, aok[p], a0, a1);
        const v8i A0 = a_half == 0 ? v8i{(int)a0.x, (int)a0.y, 0, 0, 0, 0, 0, 0}
                                   : v8i{0, 0, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
        const v8i A1 = a_half == 0 ? v8i{(int)a1.x, (int)a1.y, 0, 0, 0, 0, 0, 0}
                                   : v8i{0, 0, (int)a1.z, (int)a1.w, 0, 0, 0, 0};
        const uint2 sa = load8<FAST>(as[p], soff, sbytes, sok[p]);
        float fa[8];
        fp8x8_to_f32(sa, fa);
        const float4_t c0 = mfma_fp4(A0, B0);
        const float4_t c1 = mfma_fp4(A1, B1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t0 = 4 * (r >> 1) + (r & 1);  // scale byte for MFMA 0
          const int t1 = t0 + 2;                  // and for MFMA 1
          acc[p] = fmaf(c0[r], fa[t0] * fw[t0], acc[p]);
          acc[p] = fmaf(c1[r], fa[t1] * fw[t1], acc[p]);
        }
      }
    }
    // lanes of slices j and j^1 hold the same (row, column): add them
#pragma unroll
    for (int p = 0; p < MP; ++p) {
      acc[p] += __shfl_xor(acc[p], 16, 64);
      if ((j & 1) == 0) red[wave][2 * p + c_mloc][col] = acc[p];
    }
    __syncthreads();
    if (threadIdx.x < ROWS * 16) {
      const int rl = threadIdx.x >> 4, cc = threadIdx.x & 15;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w][rl][cc];
      const int r = r0 + rl, n = n0 + cc;
      bool ok = r < r_end && n < N;
      if (GROUPED && row_index != nullptr && ok) ok = row_index[r] >= 0 && row_index[r] < a_rows;
      if (ok) {
        const float v = s * gscale;
        if (y_bf16)
          ((uint16_t*)y)[(int64_t)r * N + n] = (uint16_t)f32_to_bf16_rne(v);
        else
          ((float*)y)[(int64_t)r * N + n] = v;
      }
    }
    __syncthreads();
  }
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <bool GROUPED>
static hipError_t launch_impl(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                              const int32_t* row_index, const int32_t* offsets, int G,
                              const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                              void* y, bool y_bf16, int64_t M, int64_t N, int64_t K,
                              int64_t a_rows, hipStream_t s) {
  constexpr int NW = 4, MP = 8;
  const bool fast = (K % 256 == 0) && aligned16(a_codes) && aligned16(a_scales) &&
                    aligned16(w_codes) && aligned16(w_scales);
  dim3 grid((unsigned)((N + 15) / 16), GROUPED ? (unsigned)G : 1u);
  if (fast)
    gemv_fp4_kernel<NW, MP, true, GROUPED><<<grid, NW * 64, 0, s>>>(
        a_codes, a_scales, gsa, row_index, offsets, w_codes, w_scales, ws2, y, y_bf16 ? 1 : 0,
        (int)M, (int)N, (int)K, (int)a_rows);
  else
    gemv_fp4_kernel<NW, MP, false, GROUPED><<<grid, NW * 64, 0, s>>>(
        a_codes, a_scales, gsa, row_index, offsets, w_codes, w_scales, ws2, y, y_bf16 ? 1 : 0,
        (int)M, (int)N, (int)K, (int)a_rows);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                       void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  return launch_impl<false>(a_codes, a_scales, gsa, nullptr, nullptr, 1, w_codes, w_scales, ws2, y,
                            y_bf16, M, N, K, M, s);
}

hipError_t launch_grouped_gemv(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                               int64_t a_rows, const int32_t* row_index, const int32_t* offsets,
                               int G, int64_t M_total, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* ws2, void* y, bool y_bf16,
                               int64_t N, int64_t K, hipStream_t s) {
  return launch_impl<true>(a_codes, a_scales, gsa, row_index, offsets, G, w_codes, w_scales, ws2,
                           y, y_bf16, M_total, N, K, a_rows, s);
}

}  // namespace nvfp4
