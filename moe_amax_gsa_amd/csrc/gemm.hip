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

// Both E4M3 scale bytes of a fragment's two blocks (low byte first) as f16,
// in one conversion (every E4M3FN value is an f16 value).
__device__ __forceinline__ half2_t scale_pair2(uint32_t two) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two, 1.0f, false);
}

// {s[I], s[I]}: the packed multiply selects the half through its operand
// selectors, so this costs no instruction.
template <int I>
__device__ __forceinline__ half2_t splat(half2_t s) {
  return __builtin_shufflevector(s, s, I, I);
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
    int y_bf16, int M, int N, int K, int gsa_rows) {
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
      const half2_t pa = scale_pair2(sa[i]), pb = scale_pair2(sb[i]);
      const half2_t fa0 = splat<0>(pa), fa1 = splat<1>(pa);
      const half2_t fb0 = splat<0>(pb), fb1 = splat<1>(pb);
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
          const float v = acc[a][b][r] * (gsa_rows ? gsa_p[row] * ws2_p[0] : gscale);
          if (y_bf16)
            ((uint16_t*)y)[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            ((float*)y)[(int64_t)row * N + col] = v;
        }
      }
}

// ------------------------------------------------------- LDS-staged tiles
// Workgroup tile (32 WM) x (32 WN), four waves.  Codes and scales are staged
// through LDS in 256-element K chunks: a chunk is one 128-byte line of codes
// and 16 scale bytes per row, fetched whole (eight lanes per line) straight
// into LDS, STAGES chunks in flight.  Each wave computes the whole tile over
// 64-element step w of every chunk -- so a wave dequantizes WM + WN
// fragments per WM * WN MFMAs -- and the four partial tiles are summed
// through LDS at the end.  Code lines sit in LDS with their 16-byte pieces
// rotated by the row (piece c of row r at slot c ^ (r & 7)), so the
// MFMA-layout reads of eight consecutive rows hit eight different bank
// groups.
template <int WM, int WN, int STAGES, int KW>
struct LdsTile {
  static constexpr int TM = 32 * WM, TN = 32 * WN, ROWS = TM + TN;
  static constexpr int THREADS = 64 * KW;
  static constexpr int CHUNK = 64 * KW;             // K elements per chunk, 64 per wave
  static constexpr int CB = CHUNK / 2, SB = CHUNK / 16;  // code, scale bytes per row
  static constexpr int PPR = CB / 16;               // 16-byte pieces per code row
  static constexpr int RPL = 1024 / CB;             // code rows per wave load
  static constexpr int SRL = 1024 / SB;             // scale rows per wave load
  static constexpr int CODE_BYTES = ROWS * CB, SCALE_BYTES = ROWS * SB;
  static constexpr int STAGE_BYTES = CODE_BYTES + SCALE_BYTES;
  static constexpr int CODE_LOADS = ROWS / (RPL * KW);  // 16-byte loads per lane per chunk
  static constexpr int SCALE_LOADS = ROWS / SRL;        // waves that fetch scales
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(ROWS % (RPL * KW) == 0 && TM % (RPL * KW) == 0, "loads must not straddle A/B");
  static_assert(ROWS % SRL == 0 && TM % SRL == 0 && SCALE_LOADS <= KW, "scale loads");
  static_assert(KW * 16 * (TN + 4) * 4 <= LDS_BYTES, "reduction slabs fit in the stages");
};

// Grouped launches: output row r belongs to group g when offsets[g] <= r <
// offsets[g + 1]; its activation row is row_index[r] (r when NULL), and
// group g's weights sit at w_codes + g N K/2, w_scales + g N K/16 with
// scale ws2[g] (dsv4/_archive/layers/grouped_linear.py, _run_impl: one
// block-scaled GEMM per group over the rows routed to it).
struct GroupArgs {
  const int32_t* row_index;
  const int32_t* offsets;
  int G;
  int a_rows;
  // SwiGLU epilogue: gate/up column groups of `gran` columns, the limit, and
  // one amax partial per workgroup (bits of the largest |h| it wrote)
  int gran;
  float limit;
  uint32_t* partials;
};

// gfx950 hands consecutive workgroups of a launch to its 8 XCDs in turn.
constexpr int GFX950_XCDS = 8;

// The tile of grouped workgroup b (1-D grid).  Work units: for each group
// g, each column tile nt and each of the group's row tiles t (ceil(rows /
// TM) of them, rows clamped to [0, M)), t fastest; they are numbered so
// that each XCD takes one contiguous run of them.  Consecutive workgroups
// on an XCD then share a weight tile -- read from HBM once, the group's
// other row tiles find it in that XCD's L2 -- and the activation rows
// (gathered, re-read by every column tile) come from L2 as well.  Every
// wave computes the same answer from the offsets, so a workgroup without a
// unit leaves as a whole.  Returns false for none; else group g, first
// output row m0, the group's end rend and column tile nt.
template <int TM>
__device__ __forceinline__ bool group_tile(const GroupArgs& ga, int M, int ntn, int& g, int& m0,
                                           int& rend, int& nt) {
  const int lane = threadIdx.x & 63;
  // the row tiles of all groups
  int total = 0;
  for (int g0 = 0; g0 < ga.G; g0 += 64) {
    const int gi = g0 + lane;
    int nti = 0;
    if (gi < ga.G) {
      const int lo = min(max(ga.offsets[gi], 0), M), hi = min(max(ga.offsets[gi + 1], 0), M);
      nti = hi > lo ? (hi - lo + TM - 1) / TM : 0;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) nti += __shfl_xor(nti, d);
    total += __builtin_amdgcn_readfirstlane(nti);
  }
  const int64_t work = (int64_t)total * ntn;
  const int64_t per = (work + GFX950_XCDS - 1) / GFX950_XCDS;
  const int64_t b = blockIdx.x, j = b / GFX950_XCDS;
  if (j >= per) return false;
  const int64_t w = (b % GFX950_XCDS) * per + j;
  if (w >= work) return false;
  // group g holds units [first * ntn, (first + nti) * ntn): the group whose
  // row-tile range holds w / ntn, from an inclusive scan of the counts
  const int slot = (int)(w / ntn);
  int base = 0;
  for (int g0 = 0; g0 < ga.G; g0 += 64) {
    const int gi = g0 + lane;
    int lo = 0, nti = 0;
    if (gi < ga.G) {
      lo = min(max(ga.offsets[gi], 0), M);
      const int hi = min(max(ga.offsets[gi + 1], 0), M);
      nti = hi > lo ? (hi - lo + TM - 1) / TM : 0;
    }
    int inc = nti;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(inc, d);
      if (lane >= d) inc += up;
    }
    const uint64_t hit = __ballot(base + inc > slot);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      g = g0 + f;
      const int n_g = __builtin_amdgcn_readlane(nti, f);
      const int first = base + __builtin_amdgcn_readlane(inc, f) - n_g;
      const int local = (int)(w - (int64_t)first * ntn);
      nt = local / n_g;
      m0 = __builtin_amdgcn_readlane(lo, f) + (local % n_g) * TM;
      rend = __builtin_amdgcn_readfirstlane(min(max(ga.offsets[g + 1], 0), M));
      return true;
    }
    base += __builtin_amdgcn_readlane(inc, 63);
  }
  return false;  // not reached: slot < total
}

template <int WM, int WN, int STAGES, int WPE, int KW, bool PIPE, bool SPLIT, bool GROUPED = false,
          bool SWIGLU = false>
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void gemm_lds_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ gsa_p, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ ws2_p, void* __restrict__ y,
    int y_bf16, int M, int N, int K, int gsa_rows, int cps, float* __restrict__ part,
    GroupArgs grp) {
  using T = LdsTile<WM, WN, STAGES, KW>;
  constexpr int TM = T::TM, TN = T::TN, LDT = TN + 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  // rows m0 .. rend - 1 of the output are this tile's (grouped: the rest of
  // the group; else all of them)
  int rend = M;
  if constexpr (GROUPED) {
    int g = 0, nt = 0;
    if (!group_tile<TM>(grp, M, (N + TN - 1) / TN, g, m0, rend, nt)) {
      if (SWIGLU && threadIdx.x == 0) grp.partials[blockIdx.x] = 0u;  // wrote no h
      return;
    }
    g = __builtin_amdgcn_readfirstlane(g);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    rend = __builtin_amdgcn_readfirstlane(rend);
    n0 = __builtin_amdgcn_readfirstlane(nt) * TN;
    w_codes += (size_t)g * N * (K / 2);
    w_scales += (size_t)g * N * (K / 16);
    ws2_p += g;
  }
  // activation row of tile row r (clamped rows: results discarded; a
  // row_index outside [0, a_rows) reads row 0 and its output is skipped)
  auto a_row = [&](int r) -> uint32_t {
    const int o = min(m0 + r, rend - 1);
    if constexpr (GROUPED) {
      if (grp.row_index == nullptr) return (uint32_t)o;
      const int ix = grp.row_index[o];
      return (ix >= 0 && ix < grp.a_rows) ? (uint32_t)ix : 0u;
    }
    return (uint32_t)o;
  };
  const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t cbytes = (uint32_t)K / 2, sbytes = (uint32_t)K / 16;
  // split z of the K range: chunks c0 .. c0 + nch - 1 (cps per split)
  const int c0 = SPLIT ? (int)blockIdx.z * cps : 0;
  const int nch = SPLIT ? min(K / T::CHUNK - c0, cps) : K / T::CHUNK;

  // code load i of wave w fills LDS rows RPL (KW i + w) .. + RPL-1: lane l
  // the row RPL (KW i + w) + l / PPR, slot l % PPR, which holds piece
  // (l % PPR) ^ (row & 7) of that row's chunk
  uint32_t csrc[T::CODE_LOADS];
#pragma unroll
  for (int i = 0; i < T::CODE_LOADS; ++i) {
    const int row = T::RPL * (KW * i + wave) + lane / T::PPR;
    const uint32_t piece = (uint32_t)((lane % T::PPR) ^ (row & 7));
    if (row < TM)
      csrc[i] = a_row(row) * cbytes + piece * 16;
    else
      csrc[i] = (uint32_t)min(n0 + row - TM, N - 1) * cbytes + piece * 16;
    csrc[i] += (uint32_t)c0 * T::CB;
  }
  // scale load of wave w < SCALE_LOADS: rows SRL w + l / (SB/16), piece l % (SB/16)
  const int srow = T::SRL * min(wave, T::SCALE_LOADS - 1) + lane / (T::SB / 16);
  const uint32_t spiece = (uint32_t)(lane % (T::SB / 16)) * 16;
  const uint32_t ssrc = (srow < TM ? a_row(srow) * sbytes
                                   : (uint32_t)min(n0 + srow - TM, N - 1) * sbytes) + spiece +
                        (uint32_t)c0 * T::SB;

  // code loads 0 .. NA-1 read A rows, the rest W rows; load i fills LDS at
  // stage + 1024 (KW i + wave)
  constexpr int NA = TM / (T::RPL * KW), NB = T::CODE_LOADS - NA;
  // The chunk advances the (uniform) base pointers; the per-lane offsets
  // stay as computed above, so issuing costs no vector instruction.
  uint32_t va[NA], vb[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) va[i] = csrc[i];
#pragma unroll
  for (int i = 0; i < NB; ++i) vb[i] = csrc[NA + i];
  auto issue = [&](int chunk, int stage) {
    const uint32_t st = smem_base + stage * T::STAGE_BYTES;
    load_lds16_run<NA>(a_codes + (size_t)chunk * T::CB, va, st + 1024 * wave, 1024 * KW);
    load_lds16_run<NB>(w_codes + (size_t)chunk * T::CB, vb, st + 1024 * (KW * NA + wave),
                       1024 * KW);
    const uint32_t sdst = st + T::CODE_BYTES + 1024 * wave;
    if (wave < TM / T::SRL)
      load_lds16(a_scales + (size_t)chunk * T::SB, ssrc, sdst);
    else if (wave < T::SCALE_LOADS)
      load_lds16(w_scales + (size_t)chunk * T::SB, ssrc, sdst);
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // LDS read offsets of this lane's fragments within a stage (wave = the
  // 64-element step of the chunk)
  const uint32_t piece = (uint32_t)(2 * wave + h);
  const uint32_t slot = (piece ^ (uint32_t)(r32 & 7)) * 16;

  if constexpr (PIPE) {
    // This wave's code fragments (16 bytes: its 64-element step of the
    // chunk) and scale pairs of every tile row, from a stage.
    // One address per stage and lane; the fragments sit at constant offsets
    // from it (folded into the LDS reads' offset fields).
    const uint32_t lane_c = (uint32_t)r32 * T::CB + slot;
    const uint32_t lane_s = T::CODE_BYTES + (uint32_t)r32 * T::SB + 4 * wave + 2 * h;
    auto read_frags = [&](int stage, uint4 (&fa)[WM], uint4 (&fb)[WN], uint32_t (&sa)[WM],
                          uint32_t (&sb)[WN]) {
      const uint8_t* pc = smem + stage * T::STAGE_BYTES + lane_c;
      const uint8_t* ps = smem + stage * T::STAGE_BYTES + lane_s;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        fa[i] = *(const uint4*)(pc + 32 * i * T::CB);
        sa[i] = *(const uint16_t*)(ps + 32 * i * T::SB);
      }
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        fb[i] = *(const uint4*)(pc + (TM + 32 * i) * T::CB);
        sb[i] = *(const uint16_t*)(ps + (TM + 32 * i) * T::SB);
      }
    };
    // scale pairs as f16 and the operands of substep 0
    half2_t sfa[WM], sfb[WN];
    half8_t A[2][WM], B[2][WN];
    auto prep = [&](const uint4 (&fa)[WM], const uint4 (&fb)[WN], const uint32_t (&sa)[WM],
                    const uint32_t (&sb)[WN]) {
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        sfa[i] = scale_pair2(sa[i]);
        A[0][i] = dequant8(fa[i].x, splat<0>(sfa[i]));
      }
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        sfb[i] = scale_pair2(sb[i]);
        B[0][i] = dequant8(fb[i].x, splat<0>(sfb[i]));
      }
    };
    // Two stages.  The wait and barrier for chunk c + 1 come before the last
    // substep of chunk c, so that substep's MFMAs run beside the next
    // chunk's fragment reads, scale conversions and first dequantization;
    // the loads of chunk c + 2 then refill the stage chunk c was read from.
    static_assert(STAGES == 2, "the pipelined loop has two stages");
    uint4 fa[WM], fb[WN];
    uint32_t sa[WM], sb[WN];
    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    read_frags(0, fa, fb, sa, sb);
    if (nch > 1) issue(1, 1);
    prep(fa, fb, sa, sb);
    for (int c = 0; c < nch; ++c) {
#pragma unroll
      for (int sub = 0; sub < 3; ++sub) {
        const int cur = sub & 1, nxt = cur ^ 1;
#pragma unroll
        for (int i = 0; i < WM; ++i) {
          const uint32_t w = sub == 0 ? fa[i].y : sub == 1 ? fa[i].z : fa[i].w;
          A[nxt][i] = dequant8(w, sub == 0 ? splat<0>(sfa[i]) : splat<1>(sfa[i]));
        }
#pragma unroll
        for (int i = 0; i < WN; ++i) {
          const uint32_t w = sub == 0 ? fb[i].y : sub == 1 ? fb[i].z : fb[i].w;
          B[nxt][i] = dequant8(w, sub == 0 ? splat<0>(sfb[i]) : splat<1>(sfb[i]));
        }
#pragma unroll
        for (int a = 0; a < WM; ++a)
#pragma unroll
          for (int b = 0; b < WN; ++b) acc[a][b] = mfma_f16(A[cur][a], B[cur][b], acc[a][b]);
#pragma unroll
        for (int g = 0; g < WM * WN; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (8 * (WM + WN) + WM * WN - 1) / (WM * WN), 0);
        }
      }
      // chunk c + 1 has landed and every wave has read chunk c's stage (at
      // the last chunk this reads a stale stage whose values are not used)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (c + 2 < nch) issue(c + 2, c & 1);
      uint4 ga[WM], gb[WN];
      uint32_t ta[WM], tb[WN];
      read_frags((c + 1) & 1, ga, gb, ta, tb);
      // substep 3 (operands in buffer 1) beside the next chunk's preparation
      half8_t A3[WM], B3[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) A3[i] = A[1][i];
#pragma unroll
      for (int i = 0; i < WN; ++i) B3[i] = B[1][i];
      prep(ga, gb, ta, tb);
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b) acc[a][b] = mfma_f16(A3[a], B3[b], acc[a][b]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (WM + WN), 0);  // the fragment reads first
#pragma unroll
      for (int g = 0; g < WM * WN; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (12 * (WM + WN) + WM * WN - 1) / (WM * WN), 0);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i) fa[i] = ga[i];
#pragma unroll
      for (int i = 0; i < WN; ++i) fb[i] = gb[i];
    }
  } else {
  #pragma unroll
    for (int s0 = 0; s0 < STAGES - 1; ++s0) issue(min(s0, nch - 1), s0);

    for (int c = 0; c < nch; ++c) {
      // chunks c+1 .. c+STAGES-2 may still be in flight: this wave issues its
      // code loads per chunk, and one scale load if it is one of the first
      // SCALE_LOADS waves
      constexpr int W_SCALE = (STAGES - 2) * (T::CODE_LOADS + 1);
      constexpr int W_CODE = (STAGES - 2) * T::CODE_LOADS;
      if (wave < T::SCALE_LOADS)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W_SCALE) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W_CODE) : "memory");
      lds_barrier();
      issue(min(c + STAGES - 1, nch - 1), (c + STAGES - 1) % STAGES);

      const uint8_t* st = smem + (c % STAGES) * T::STAGE_BYTES;
      uint4 fa[WM], fb[WN];
      uint32_t sa[WM], sb[WN];
  #pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int row = 32 * i + r32;
        fa[i] = *(const uint4*)(st + row * T::CB + slot);
        sa[i] = *(const uint16_t*)(st + T::CODE_BYTES + row * T::SB + 4 * wave + 2 * h);
      }
  #pragma unroll
      for (int i = 0; i < WN; ++i) {
        const int row = TM + 32 * i + r32;
        fb[i] = *(const uint4*)(st + row * T::CB + slot);
        sb[i] = *(const uint16_t*)(st + T::CODE_BYTES + row * T::SB + 4 * wave + 2 * h);
      }
      half2_t sfa[WM], sfb[WN];
  #pragma unroll
      for (int i = 0; i < WM; ++i) sfa[i] = scale_pair2(sa[i]);
  #pragma unroll
      for (int i = 0; i < WN; ++i) sfb[i] = scale_pair2(sb[i]);
      half8_t A[2][WM], B[2][WN];
  #pragma unroll
      for (int i = 0; i < WM; ++i) A[0][i] = dequant8(fa[i].x, splat<0>(sfa[i]));
  #pragma unroll
      for (int i = 0; i < WN; ++i) B[0][i] = dequant8(fb[i].x, splat<0>(sfb[i]));
  #pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const int cur = sub & 1, nxt = cur ^ 1;
        if (sub < 3) {
  #pragma unroll
          for (int i = 0; i < WM; ++i) {
            const uint32_t w = sub == 0 ? fa[i].y : sub == 1 ? fa[i].z : fa[i].w;
            A[nxt][i] = dequant8(w, sub == 0 ? splat<0>(sfa[i]) : splat<1>(sfa[i]));
          }
  #pragma unroll
          for (int i = 0; i < WN; ++i) {
            const uint32_t w = sub == 0 ? fb[i].y : sub == 1 ? fb[i].z : fb[i].w;
            B[nxt][i] = dequant8(w, sub == 0 ? splat<0>(sfb[i]) : splat<1>(sfb[i]));
          }
        }
  #pragma unroll
        for (int a = 0; a < WM; ++a)
  #pragma unroll
          for (int b = 0; b < WN; ++b) acc[a][b] = mfma_f16(A[cur][a], B[cur][b], acc[a][b]);
        if (sub < 3) {
          // one MFMA, then a share of the next substep's dequantization
  #pragma unroll
          for (int g = 0; g < WM * WN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, (8 * (WM + WN) + WM * WN - 1) / (WM * WN), 0);
          }
        }
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // reduce the KW partial tiles one 16-row slab at a time (result registers
  // 8q..8q+7 of MFMA tile row a hold rows 32a + 16q + [0, 16))
  float* red = (float*)smem;
  const float gscale = gsa_p[0] * ws2_p[0];
  float* slab = red + (size_t)wave * 16 * LDT;
  float hmax = 0.f;  // SWIGLU: the largest |h| this thread wrote
  // is output row `row` written (inside the tile's group, valid row_index)
  auto live_row = [&](int row) -> bool {
    bool live = row < rend;
    if constexpr (GROUPED) {
      if (live && grp.row_index != nullptr) {
        const int ix = grp.row_index[row];
        live = ix >= 0 && ix < grp.a_rows;
      }
    }
    return live;
  };
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
      if constexpr (SWIGLU) {
        // h column n0 / 2 + hc pairs the tile's gate column cg with the up
        // column cg + gran (the tile starts on a whole number of pairs)
        const int lg = __builtin_ctz(grp.gran);
        for (int e = threadIdx.x; e < 16 * (TN / 2); e += T::THREADS) {
          const int rr = e / (TN / 2), hc = e % (TN / 2);
          const int cg = ((hc >> lg) << (lg + 1)) + (hc & (grp.gran - 1)), cu = cg + grp.gran;
          float vg = red[rr * LDT + cg], vu = red[rr * LDT + cu];
#pragma unroll
          for (int w = 1; w < KW; ++w) {
            vg += red[(w * 16 + rr) * LDT + cg];
            vu += red[(w * 16 + rr) * LDT + cu];
          }
          const int row = m0 + a * 32 + q * 16 + rr;
          if (n0 + cg < N && live_row(row)) {
            const float hv = swiglu1(vg * gscale, vu * gscale, grp.limit);
            ((float*)y)[(int64_t)row * (N / 2) + n0 / 2 + hc] = hv;
            hmax = fmaxf(hmax, fabsf(hv));
          }
        }
      } else {
        for (int e = threadIdx.x; e < 16 * TN; e += T::THREADS) {
          const int rr = e / TN, cc = e % TN;
          float v = red[rr * LDT + cc];
#pragma unroll
          for (int w = 1; w < KW; ++w) v += red[(w * 16 + rr) * LDT + cc];
          const int row = m0 + a * 32 + q * 16 + rr, col = n0 + cc;
          if (col < N && live_row(row)) {
            if (SPLIT) {  // the raw partial sum of this split
              part[((int64_t)blockIdx.z * M + row) * N + col] = v;
            } else {
              const float o = v * (gsa_rows ? gsa_p[row] * ws2_p[0] : gscale);
              if (y_bf16)
                ((uint16_t*)y)[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(o);
              else
                ((float*)y)[(int64_t)row * N + col] = o;
            }
          }
        }
      }
      __syncthreads();
    }
  }
  if constexpr (SWIGLU) {  // the workgroup's largest |h| (reusing the slab LDS)
    uint32_t* wmax = (uint32_t*)smem;
    const uint32_t m = wave_max_u32(__float_as_uint(hmax));
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mm = 0;
      for (int w = 0; w < KW; ++w) mm = max(mm, wmax[w]);
      grp.partials[blockIdx.x] = mm;
    }
  }
}

// Sum of the split-K partials in split order (deterministic), times the
// epilogue scale: one output per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t MN, int N,
                                                            const float* __restrict__ gsa_p,
                                                            const float* __restrict__ ws2_p,
                                                            int gsa_rows, void* __restrict__ y,
                                                            int y_bf16) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= MN) return;
  // every split's load in flight at once, then the sum in split order
  float p[GEMM_MAX_SPLITS];
#pragma unroll
  for (int z = 0; z < GEMM_MAX_SPLITS; ++z) p[z] = z < splits ? part[(int64_t)z * MN + e] : 0.0f;
  float v = p[0];
#pragma unroll
  for (int z = 1; z < GEMM_MAX_SPLITS; ++z)
    if (z < splits) v += p[z];
  const float sc = (gsa_rows ? gsa_p[e / N] : gsa_p[0]) * ws2_p[0];
  const float o = v * sc;
  if (y_bf16)
    ((uint16_t*)y)[e] = (uint16_t)f32_to_bf16_rne(o);
  else
    ((float*)y)[e] = o;
}

// ------------------------------------------------------- wide tiles
// Workgroup tile 256 x 256 for shapes with enough such tiles to fill the
// chip.  Eight waves in a 2 (rows) x 4 (columns) arrangement each own a
// 128 x 64 output block over the whole K range, so no partial tiles are
// summed across waves.  Both operands' 256-element chunks (one 128-byte code
// line and 16 scale bytes per row, 512 rows) are staged through LDS as in
// the kernel above, two stages; a wave reads and dequantizes its own 4 + 2
// fragments per 64-element step and runs 8 MFMAs per 16 elements.  Per flop
// this moves a third of the bytes of the 128 x 64 tile.
struct WideTile {
  static constexpr int TM = 256, TN = 256, ROWS = TM + TN, KW = 8, THREADS = 64 * KW;
  static constexpr int CHUNK = 256, CB = 128, SB = 16;
  static constexpr int CODE_BYTES = ROWS * CB;                // 64 KiB
  static constexpr int STAGE_BYTES = CODE_BYTES + ROWS * SB;  // + 8 KiB of scales
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int CODE_LOADS = ROWS / (8 * KW);  // a load covers 8 rows: 8 per wave
  static constexpr int NA = TM / (8 * KW);             // the first 4 read A rows
};

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_wide_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ gsa_p, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ ws2_p, void* __restrict__ y,
    int y_bf16, int M, int N, int K, int gsa_rows) {
  using T = WideTile;
  constexpr int WM = 4, WN = 2, NA = T::NA, NB = T::CODE_LOADS - T::NA;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int r32 = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.y * T::TM, n0 = blockIdx.x * T::TN;
  const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t cbytes = (uint32_t)K / 2, sbytes = (uint32_t)K / 16;
  const int nch = K / T::CHUNK;

  // code load i of wave w: LDS rows 8 (KW i + w) + l / 8, lane l filling
  // slot l % 8 with piece (l % 8) ^ (row & 7) of the row's chunk line
  uint32_t va[NA], vb[NB];
#pragma unroll
  for (int i = 0; i < T::CODE_LOADS; ++i) {
    const int row = 8 * (T::KW * i + wave) + lane / 8;
    const uint32_t off = (uint32_t)((lane % 8) ^ (row & 7)) * 16;
    if (i < NA)
      va[i] = (uint32_t)min(m0 + row, M - 1) * cbytes + off;  // clamped rows: discarded
    else
      vb[i - NA] = (uint32_t)min(n0 + row - T::TM, N - 1) * cbytes + off;
  }
  // scale load of wave w: rows 64 w + l (A rows for w < 4), 16 bytes each
  const int srow = 64 * wave + lane;
  const uint32_t ssrc = srow < T::TM ? (uint32_t)min(m0 + srow, M - 1) * sbytes
                                     : (uint32_t)min(n0 + srow - T::TM, N - 1) * sbytes;
  auto issue = [&](int chunk, int stage) {
    const uint32_t st = smem_base + stage * T::STAGE_BYTES;
    load_lds16_run<NA>(a_codes + (size_t)chunk * T::CB, va, st + 1024 * wave, 1024 * T::KW);
    load_lds16_run<NB>(w_codes + (size_t)chunk * T::CB, vb, st + 1024 * (T::KW * NA + wave),
                       1024 * T::KW);
    const uint32_t sdst = st + T::CODE_BYTES + 1024 * wave;
    if (wave < T::TM / 64)
      load_lds16(a_scales + (size_t)chunk * T::SB, ssrc, sdst);
    else
      load_lds16(w_scales + (size_t)chunk * T::SB, ssrc, sdst);
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // this lane's rows of the stage: A rows 128 wm + 32 i + r32, W rows
  // 256 + 64 wn + 32 j + r32 (all with row & 7 == r32 & 7)
  const uint32_t a_row0 = (uint32_t)(128 * wm + r32), b_row0 = (uint32_t)(T::TM + 64 * wn + r32);

  issue(0, 0);
  for (int c = 0; c < nch; ++c) {
    // chunk c has landed everywhere, and every wave is done with the stage
    // chunk c + 1 will refill
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (c + 1 < nch) issue(c + 1, (c + 1) & 1);
    const uint8_t* st = smem + (c & 1) * T::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // step s of the chunk: lane half h owns its pieces 2s + h
      const uint32_t slot = (uint32_t)(((2 * s + h) ^ (r32 & 7)) * 16);
      uint4 fa[WM], fb[WN];
      half2_t sfa[WM], sfb[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const uint32_t row = a_row0 + 32 * i;
        fa[i] = *(const uint4*)(st + row * T::CB + slot);
        sfa[i] = scale_pair2(*(const uint16_t*)(st + T::CODE_BYTES + row * T::SB + 4 * s + 2 * h));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint32_t row = b_row0 + 32 * j;
        fb[j] = *(const uint4*)(st + row * T::CB + slot);
        sfb[j] = scale_pair2(*(const uint16_t*)(st + T::CODE_BYTES + row * T::SB + 4 * s + 2 * h));
      }
      half8_t A[2][WM], B[2][WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) A[0][i] = dequant8(fa[i].x, splat<0>(sfa[i]));
#pragma unroll
      for (int j = 0; j < WN; ++j) B[0][j] = dequant8(fb[j].x, splat<0>(sfb[j]));
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const int cur = sub & 1, nxt = cur ^ 1;
        if (sub < 3) {
#pragma unroll
          for (int i = 0; i < WM; ++i) {
            const uint32_t w = sub == 0 ? fa[i].y : sub == 1 ? fa[i].z : fa[i].w;
            A[nxt][i] = dequant8(w, sub == 0 ? splat<0>(sfa[i]) : splat<1>(sfa[i]));
          }
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const uint32_t w = sub == 0 ? fb[j].y : sub == 1 ? fb[j].z : fb[j].w;
            B[nxt][j] = dequant8(w, sub == 0 ? splat<0>(sfb[j]) : splat<1>(sfb[j]));
          }
        }
#pragma unroll
        for (int a = 0; a < WM; ++a)
#pragma unroll
          for (int b = 0; b < WN; ++b) acc[a][b] = mfma_f16(A[cur][a], B[cur][b], acc[a][b]);
        if (sub < 3) {
#pragma unroll
          for (int g = 0; g < WM * WN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, (8 * (WM + WN) + WM * WN - 1) / (WM * WN), 0);
          }
        }
      }
    }
  }

  // each wave stores its own block: result register r of MFMA tile (a, b)
  // is row 32a + 8(r/4) + 4h + r%4, column 32b + r32 of the block
  const float gscale = gsa_p[0] * ws2_p[0];
  const float w2 = ws2_p[0];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + 128 * wm + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= M) continue;
      const float sc = gsa_rows ? gsa_p[row] * w2 : gscale;
#pragma unroll
      for (int b = 0; b < WN; ++b) {
        const int col = n0 + 64 * wn + 32 * b + r32;
        if (col >= N) continue;
        const float o = acc[a][b][r] * sc;
        if (y_bf16)
          ((uint16_t*)y)[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(o);
        else
          ((float*)y)[(int64_t)row * N + col] = o;
      }
    }
}

static hipError_t launch_wide(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                              const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                              void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s,
                              bool gsa_rows) {
  using T = WideTile;
  static_assert(T::LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  // the loop loads chunk 0 unconditionally: K must hold whole chunks
  if (K < T::CHUNK || K % T::CHUNK != 0) return hipErrorInvalidValue;
  static unsigned char done[64];
  const hipError_t attr = allow_dynamic_lds((const void*)gemm_wide_kernel, T::LDS_BYTES, done);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)((N + T::TN - 1) / T::TN), (unsigned)((M + T::TM - 1) / T::TM));
  gemm_wide_kernel<<<grid, T::THREADS, T::LDS_BYTES, s>>>(a_codes, a_scales, gsa, w_codes,
                                                          w_scales, ws2, y, y_bf16 ? 1 : 0,
                                                          (int)M, (int)N, (int)K,
                                                          gsa_rows ? 1 : 0);
  return hipGetLastError();
}

template <int WM, int WN, int STAGES, int WPE, int KW, bool PIPE = false>
hipError_t launch_lds(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                      const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2, void* y,
                      bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s,
                      bool gsa_rows = false, int splits = 1, float* part = nullptr,
                      bool reduce = true) {
  using T = LdsTile<WM, WN, STAGES, KW>;
  static_assert(T::LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  const int nch = (int)(K / T::CHUNK);
  // the prologue loads chunk 0 (and chunk min(s, nch - 1) for deeper
  // stages) unconditionally: K must hold whole chunks, at least one
  if (nch < 1 || K % T::CHUNK != 0) return hipErrorInvalidValue;
  const int cps = (nch + splits - 1) / splits;
  splits = (nch + cps - 1) / cps;  // every split has at least one chunk
  const dim3 grid((unsigned)((N + T::TN - 1) / T::TN), (unsigned)((M + T::TM - 1) / T::TM),
                  (unsigned)splits);
  if (splits == 1 || part == nullptr) {
    static unsigned char done[64];
    const hipError_t attr = allow_dynamic_lds(
        (const void*)gemm_lds_kernel<WM, WN, STAGES, WPE, KW, PIPE, false>, T::LDS_BYTES, done);
    if (attr != hipSuccess) return attr;
    gemm_lds_kernel<WM, WN, STAGES, WPE, KW, PIPE, false>
        <<<dim3(grid.x, grid.y), T::THREADS, T::LDS_BYTES, s>>>(
            a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16 ? 1 : 0, (int)M, (int)N,
            (int)K, gsa_rows ? 1 : 0, nch, nullptr, GroupArgs{});
    return hipGetLastError();
  }
  static unsigned char done[64];
  const hipError_t attr = allow_dynamic_lds(
      (const void*)gemm_lds_kernel<WM, WN, STAGES, WPE, KW, PIPE, true>, T::LDS_BYTES, done);
  if (attr != hipSuccess) return attr;
  gemm_lds_kernel<WM, WN, STAGES, WPE, KW, PIPE, true><<<grid, T::THREADS, T::LDS_BYTES, s>>>(
      a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16 ? 1 : 0, (int)M, (int)N, (int)K,
      gsa_rows ? 1 : 0, cps, part, GroupArgs{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !reduce) return e;
  const int64_t MN = M * N;
  splitk_reduce_kernel<<<(unsigned)((MN + 255) / 256), 256, 0, s>>>(
      part, splits, MN, (int)N, gsa, ws2, gsa_rows ? 1 : 0, y, y_bf16 ? 1 : 0);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Split-K plan for the staged kernel: with few output tiles (at most half a
// tile per CU) the K range is cut into up to 16 splits, about one
// workgroup per CU.  (Measured on MI355X at K = 7168, M = 64 to 128: about
// two workgroups per CU took 10-21% longer from 24 tiles up, 64 x 1536
// 13.9 against 16.1 us, 128 x 2048 17.5 against 22.1 us, 128 x 4096 21.6
// against 24.3 us, and the same at 6 tiles, where both take 16.)  Returns
// the split count (1: none).
static int gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((N + 63) / 64) * ((M + 127) / 128);
  const int64_t nch = K / 256;
  if (2 * tiles > device_cu_count() || nch < 2) return 1;
  int64_t sp = device_cu_count() / tiles;
  sp = sp < GEMM_MAX_SPLITS ? sp : GEMM_MAX_SPLITS;
  sp = sp < nch ? sp : nch;
  const int64_t cps = (nch + sp - 1) / sp;
  return (int)((nch + cps - 1) / cps);
}

static bool gemm_staged_ok(const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales, int64_t M, int64_t N,
                           int64_t K) {
  const bool fast = (K % 64 == 0) && (((uintptr_t)a_codes | (uintptr_t)w_codes) & 15u) == 0 &&
                    (((uintptr_t)a_scales | (uintptr_t)w_scales) & 1u) == 0;
  // the staged kernel takes whole 256-element chunks and 32-bit row offsets
  return fast && K % 256 == 0 && K >= 256 && M * (K / 2) < (1ll << 31) &&
         N * (K / 2) < (1ll << 31);
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K % 256 != 0 || K < 256) return 0;
  const int sp = gemm_splits(M, N, K);
  return sp > 1 ? (size_t)sp * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                       void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s,
                       bool gsa_rows, void* ws, size_t ws_bytes, int* partial_splits) {
  if (partial_splits) *partial_splits = 0;
  const bool fast = (K % 64 == 0) && (((uintptr_t)a_codes | (uintptr_t)w_codes) & 15u) == 0 &&
                    (((uintptr_t)a_scales | (uintptr_t)w_scales) & 1u) == 0;
  const bool big = gemm_staged_ok(a_codes, a_scales, w_codes, w_scales, M, N, K);
  if (big) {
    const int sp = gemm_splits(M, N, K);
    if (sp > 1 && ws != nullptr && ((uintptr_t)ws & 15u) == 0 &&
        ws_bytes >= (size_t)sp * M * N * sizeof(float)) {
      if (partial_splits) *partial_splits = sp;  // the caller adds the partials
      return launch_lds<4, 2, 2, 2, 4>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16,
                                       M, N, K, s, gsa_rows, sp, (float*)ws,
                                       partial_splits == nullptr);
    }
    // 128 x 64 tiles.  At most one tile per CU: eight waves split each
    // 512-element chunk (two waves per SIMD) and the next chunk's fragment
    // reads and first dequantization run under the current chunk's last
    // MFMAs.  More tiles: four waves, two workgroups per CU.
    // 256 x 256 tiles where they keep at least three quarters of the CUs busy
    const int64_t wide = ((N + 255) / 256) * ((M + 255) / 256);
    if (4 * wide >= 3 * (int64_t)device_cu_count())
      return launch_wide(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16, M, N, K, s,
                         gsa_rows);
    const int64_t tiles = ((N + 63) / 64) * ((M + 127) / 128);
    if (tiles <= device_cu_count() && K % 512 == 0)
      return launch_lds<4, 2, 2, 2, 8, true>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y,
                                             y_bf16, M, N, K, s, gsa_rows);
    return launch_lds<4, 2, 2, 2, 4>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16, M,
                                     N, K, s, gsa_rows);
  }
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128));
  if (fast)
    gemm_f16_kernel<true><<<grid, 256, 0, s>>>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y,
                                               y_bf16 ? 1 : 0, (int)M, (int)N, (int)K,
                                               gsa_rows ? 1 : 0);
  else
    gemm_f16_kernel<false><<<grid, 256, 0, s>>>(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y,
                                                y_bf16 ? 1 : 0, (int)M, (int)N, (int)K,
                                                gsa_rows ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4

namespace nvfp4 {

// Grouped tiled linear for groups of many rows: the staged kernel over the
// row tiles of every group (the tile count is known on the device only, so
// the grid covers the most there can be, ceil(M_total / TM) + G row tiles,
// and the workgroups past the real count leave at once).
bool grouped_gemm_supported(const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* w_codes, const uint8_t* w_scales, int64_t a_rows,
                            int64_t M_total, int G, int64_t N, int64_t K) {
  return gemm_staged_ok(a_codes, a_scales, w_codes, w_scales, a_rows, N, K) &&
         grouped_tile_blocks(M_total, G, N) <= 2147483647ll;
}

template <int WM, int WN, int KW, bool PIPE, bool SWIGLU>
static hipError_t launch_grouped_tiles(const uint8_t* a_codes, const uint8_t* a_scales,
                                       const float* gsa, const GroupArgs& ga, int64_t M_total,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const float* ws2, void* y, bool y_bf16, int64_t N,
                                       int64_t K, hipStream_t s) {
  using T = LdsTile<WM, WN, 2, KW>;
  static_assert(T::LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
  const int64_t blocks = grouped_tile_blocks(M_total, ga.G, N);
  static unsigned char done[64];
  const hipError_t attr = allow_dynamic_lds(
      (const void*)gemm_lds_kernel<WM, WN, 2, 2, KW, PIPE, false, true, SWIGLU>, T::LDS_BYTES,
      done);
  if (attr != hipSuccess) return attr;
  gemm_lds_kernel<WM, WN, 2, 2, KW, PIPE, false, true, SWIGLU>
      <<<dim3((unsigned)blocks), T::THREADS, T::LDS_BYTES, s>>>(
          a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16 ? 1 : 0, (int)M_total,
          (int)N, (int)K, 0, (int)(K / T::CHUNK), nullptr, ga);
  return hipGetLastError();
}

// 64 x 128 tiles: a group's last row tile is on average half empty (the
// group sizes are known on the device only), and 64-row tiles waste half as
// many rows as 128-row ones.  As launch_gemm: eight waves per tile while the
// tiles are no more than the CUs, else four (two workgroups per CU).
template <bool SWIGLU>
static hipError_t launch_grouped_any(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const float* gsa, const GroupArgs& ga, int64_t M_total,
                                     const uint8_t* w_codes, const uint8_t* w_scales,
                                     const float* ws2, void* y, bool y_bf16, int64_t N, int64_t K,
                                     hipStream_t s) {
  const int64_t tiles = ((M_total + 63) / 64) * ((N + 127) / 128);
  if (tiles <= device_cu_count() && K % 512 == 0)
    return launch_grouped_tiles<2, 4, 8, true, SWIGLU>(a_codes, a_scales, gsa, ga, M_total,
                                                       w_codes, w_scales, ws2, y, y_bf16, N, K, s);
  return launch_grouped_tiles<2, 4, 4, false, SWIGLU>(a_codes, a_scales, gsa, ga, M_total,
                                                      w_codes, w_scales, ws2, y, y_bf16, N, K, s);
}

int64_t grouped_tile_blocks(int64_t M_total, int G, int64_t N) {
  const int64_t b = ((M_total + 63) / 64 + G) * ((N + 127) / 128);
  return (b + GFX950_XCDS - 1) / GFX950_XCDS * GFX950_XCDS;
}

hipError_t launch_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                               int64_t a_rows, const int32_t* row_index, const int32_t* offsets,
                               int G, int64_t M_total, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* ws2, void* y, bool y_bf16,
                               int64_t N, int64_t K, hipStream_t s) {
  const GroupArgs ga{row_index, offsets, G, (int)a_rows, 0, 0.f, nullptr};
  return launch_grouped_any<false>(a_codes, a_scales, gsa, ga, M_total, w_codes, w_scales, ws2, y,
                                   y_bf16, N, K, s);
}

hipError_t launch_grouped_gemm_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                      const float* gsa, int64_t a_rows, const int32_t* row_index,
                                      const int32_t* offsets, int G, int64_t M_total,
                                      const uint8_t* w_codes, const uint8_t* w_scales,
                                      const float* ws2, float* h, int64_t N, int64_t K, int gran,
                                      float limit, uint32_t* partials, hipStream_t s) {
  const GroupArgs ga{row_index, offsets, G, (int)a_rows, gran, limit, partials};
  return launch_grouped_any<true>(a_codes, a_scales, gsa, ga, M_total, w_codes, w_scales, ws2, h,
                                  false, N, K, s);
}

}  // namespace nvfp4
