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
// waves split K in groups of S super-chunks of 256 elements (128 bytes per
// row, two MFMAs each) and issue a whole group's weight loads before using
// any.  A lane's 32 bytes of a super-chunk are K slice j of MFMA 0 (first 16
// bytes) and MFMA 1 (next 16).  Slice j of MFMA h spans blocks 16c + 4j + 2h
// and +1, so A row i (slot s = i % 8) takes the half s % 2 of slice s / 2.
// Result row i of MFMA h is block 16c + 8(j%2) + 4(r/2) + 2h + (r%2) for lane
// slice j and register r, whose two scale bytes sit in one 8-byte word per
// row at byte 16c + 8(j%2).
//
// Fused mode (nvfp4_linear_run): for a few activation rows the whole step
// amax -> gsa -> quantize -> linear is one kernel.  Every workgroup loads the
// entire (small) activation, computes its exact maximum itself -- there is no
// reduction across workgroups, so no workgroup ever waits for another -- and
// quantizes it into LDS while its first weight loads are in flight.
// Workgroup (0, 0) also writes gsa, codes and scales to memory.
#include "device.hpp"
#include "launch.hpp"
#include "router.hpp"

namespace nvfp4 {

typedef __attribute__((ext_vector_type(8))) int v8i;

constexpr int GEMV_MAX_WAVES = 8;
enum { MODE_PLAIN = 0, MODE_GROUPED = 1, MODE_RUN = 2 };

struct GemvArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* gsa;
  const int32_t* row_index;
  const int32_t* offsets;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* ws2;
  void* y;
  int y_bf16, M, N, K, a_rows;
  // MODE_RUN: the activation and where workgroup (0, 0) stores its quantization
  const void* x;
  float* gsa_out;
  uint8_t* codes_out;
  uint8_t* scales_out;
  // gemv_ring_kernel with SwiGLU: gate/up group width, the SwiGLU limit
  // (<= 0: none), and one amax partial (bits of a non-negative float) per
  // workgroup
  int gran;
  float limit;
  uint32_t* partials;
  // plain mode, and the ring over one group of all rows on given codes:
  // gsa holds one global scale per activation row (gsa[m])
  int gsa_rows;
  // grouped ring: G groups in all; when the grid has fewer rows of
  // workgroups than groups, workgroup row y serves the y-th group that has
  // rows (found on the device from the offsets)
  int groups;
  // gemv_ring_kernel quantizing its own activation rows from x (RING_Q_*):
  // the amax partials of an earlier launch whose maximum gives gsa
  const uint32_t* parts_in;
  int nparts_in;
  // the dense router's choice after the gate linear, in the same launch
  // (the kernels' ROUTER flag): k experts per row, the bias (or NULL), the
  // outputs, and the ticket counter in the workspace
  int router_k;
  const float* router_bias;
  int32_t* router_idx;
  float* router_score;
  uint32_t* router_count;
};

// The gate linear's last workgroup chooses the experts.  Every workgroup
// writes its logits to args.y with device-coherent stores (written through
// past its XCD's L2, store_logit), waits until they have completed, and then
// takes a ticket from a counter (a device-scope vector atomic); the one that
// takes the last ticket reads every logit with device-coherent loads, runs
// the choice for every row and sets the counter back to zero for the next
// call.  No workgroup waits for another: each exits once it has its ticket.
// (A device-scope fence would write back and invalidate whole L2s in every
// workgroup instead.)
__device__ __forceinline__ void store_logit(const GemvArgs& args, int64_t e, float v) {
  __hip_atomic_store((float*)args.y + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void router_finish(const GemvArgs& args) {
  __shared__ int last;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's logits are written
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t n = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t t = __hip_atomic_fetch_add(args.router_count, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    last = t == n - 1;
  }
  __syncthreads();
  if (!last) return;  // uniform over the workgroup
  router_choose_rows<true>((const float*)args.y, args.M, args.N, args.router_k,
                           args.router_bias, args.router_idx, args.router_score);
  if (threadIdx.x == 0)
    __hip_atomic_store(args.router_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where gemv_ring_kernel's activation rows come from.
enum {
  RING_Q_CODES = 0,  // codes and scales in memory (a_codes, a_scales, gsa)
  RING_Q_X = 1,      // quantized in the workgroup from x (a_rows x K), gsa
                     // from the amax of all of x, which every workgroup takes
  RING_Q_PARTS = 2,  // quantized in the workgroup from x, gsa from the maximum
                     // of parts_in (an earlier launch's first amax phase)
};

__device__ __forceinline__ float4_t mfma_fp4(v8i a, v8i b) {
  const float4_t z = {0.f, 0.f, 0.f, 0.f};
  // cbsz = blgp = 4: both operands E2M1; operand scale bytes 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 0, 127, 0, 127);
}

// 32 code bytes of a row at byte offset off, zero outside [0, rowbytes) or
// when !ok.  FAST: whole super-chunks inside rows, 16-byte aligned.
// Otherwise 8-byte pieces (rows are 8-byte aligned since K % 16 == 0).
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

// Streaming 16-byte load: weights are read once per call, so they need not
// stay in the vector L1.
__device__ __forceinline__ uint4 ldg_nt16(const uint8_t* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 8 bytes, nontemporal: a weight row's scales, read once per call like its
// codes.
__device__ __forceinline__ uint2 ldg_nt8(const uint8_t* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
  return make_uint2(v.x, v.y);
}

// Weight codes and scales of S super-chunks (group cg) for this lane.  FAST:
// unconditional loads of a clamped, always valid chunk -- chunks past the
// end are skipped by the (wave-uniform) compute loop.  A branch around the
// loads would make the compiler drain every outstanding load at its merge.
template <int S, bool FAST>
__device__ __forceinline__ void load_w_group(const uint8_t* wrow, const uint8_t* wsrow, int cg,
                                             int nsc, int j, int64_t cbytes, int64_t sbytes,
                                             uint4 wb0[S], uint4 wb1[S], uint2 wsb[S]) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = FAST ? min(cg * S + s, nsc - 1) : cg * S + s;
    const bool ok = FAST || c < nsc;
    if (FAST) {
      wb0[s] = ldg_nt16(wrow + (int64_t)c * 128 + 32 * j);
      wb1[s] = ldg_nt16(wrow + (int64_t)c * 128 + 32 * j + 16);
    } else {
      load32<FAST>(wrow, (int64_t)c * 128 + 32 * j, cbytes, ok, wb0[s], wb1[s]);
    }
    wsb[s] = FAST ? ldg_nt8(wsrow + (int64_t)c * 16 + 8 * (j & 1))
                  : load8<FAST>(wsrow, (int64_t)c * 16 + 8 * (j & 1), sbytes, ok);
  }
}

// S super-chunks per wave group; MP activation-row pairs per pass (pairs
// past the last row are skipped); BPT activation blocks per thread in
// MODE_RUN (the activation is held in registers between its amax and its
// quantization).
template <int S, int MP, bool FAST, int MODE, bool XBF16, int BPT, bool ROUTER = false>
__global__ __launch_bounds__(GEMV_MAX_WAVES * 64) void gemv_fp4_kernel(const GemvArgs args) {
  constexpr int ROWS = 2 * MP;
  __shared__ float red[GEMV_MAX_WAVES][ROWS][16];
  __shared__ float amax_red[GEMV_MAX_WAVES];
  extern __shared__ __attribute__((aligned(16))) uint8_t act_lds[];

  const int NW = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, j = lane >> 4;
  const int M = args.M, N = args.N, K = args.K;
  const int n0 = blockIdx.x * 16;
  const int g = MODE == MODE_GROUPED ? (int)blockIdx.y : 0;
  int r_begin = 0, r_end = M;
  if (MODE == MODE_GROUPED) {
    r_begin = max(args.offsets[g], 0);
    r_end = min(args.offsets[g + 1], M);
    if (r_begin >= r_end) return;  // uniform over the workgroup
  }
  const int64_t cbytes = K / 2, sbytes = K / 16;
  const int64_t n_here = (n0 + col < N) ? n0 + col : n0;  // clamp: results discarded
  const uint8_t* wrow = args.w_codes + ((int64_t)g * N + n_here) * cbytes;
  const uint8_t* wsrow = args.w_scales + ((int64_t)g * N + n_here) * sbytes;
  const int nsc = (K + 255) / 256;

  // A operand: lane row i = col -> local row 2p + (i / 8), slot s = i % 8,
  // carries data only when s / 2 == j, in half s % 2.
  const int a_mloc = col >> 3, a_half = col & 1;
  const bool a_has = ((col & 7) >> 1) == j;
  // Result: lane rows 4j .. 4j+3 belong to local row 2p + j / 2.
  const int c_mloc = j >> 1;

  const uint8_t* lds_codes = act_lds;
  const uint8_t* lds_scales = act_lds + (size_t)M * cbytes;

  for (int r0 = r_begin; r0 < r_end; r0 += ROWS) {
    // MODE_RUN: the activation blocks this thread quantizes, loaded first so
    // that waiting for them does not wait for the weight loads issued next.
    const int64_t nblk = (int64_t)M * (K / 16);
    float xv[BPT][16];
    bool xok[BPT];
    if (MODE == MODE_RUN) {
      // unconditional loads (index clamped): a branch here would make the
      // compiler wait for them before issuing the weight loads below
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        const int64_t b = threadIdx.x + (int64_t)q * blockDim.x;
        xok[q] = b < nblk;
        load_block16<XBF16>(args.x, xok[q] ? b : nblk - 1, xv[q]);
      }
      __builtin_amdgcn_sched_barrier(0);  // activation loads before weight loads
    }

    // first weight group of this wave
    int cg = wave;
    uint4 wb0[S], wb1[S];
    uint2 wsb[S];
    load_w_group<S, FAST>(wrow, wsrow, cg, nsc, j, cbytes, sbytes, wb0, wb1, wsb);

    float gsa_v;
    if (MODE == MODE_RUN) {
      float m = 0.f;
#pragma unroll
      for (int q = 0; q < BPT; ++q)
        if (xok[q]) m = fmaxf(m, block_absmax16(xv[q]));
      m = wave_max_f32(m);
      if (lane == 0) amax_red[wave] = m;
      lds_barrier();
      float mm = 0.f;
      for (int w = 0; w < NW; ++w) mm = fmaxf(mm, amax_red[w]);
      gsa_v = gsa_from_amax(mm);
      const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        const int64_t b = threadIdx.x + (int64_t)q * blockDim.x;
        if (xok[q]) {
          uint32_t lo, hi, sf;
          quantize_vals16(xv[q], gsa_v, lo, hi, sf);
          ((uint2*)act_lds)[b] = make_uint2(lo, hi);
          act_lds[(size_t)M * cbytes + b] = (uint8_t)sf;
          if (writer) {
            ((uint2*)args.codes_out)[b] = make_uint2(lo, hi);
            args.scales_out[b] = (uint8_t)sf;
          }
        }
      }
      if (writer && threadIdx.x == 0) args.gsa_out[0] = gsa_v;
      lds_barrier();
    } else {
      gsa_v = args.gsa[0];
    }
    const float gscale = gsa_v * args.ws2[g];

    // activation rows of this pass
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
      if (MODE == MODE_GROUPED && args.row_index != nullptr) {
        rowa = args.row_index[rowa];
        rowc = args.row_index[rowc];
        // an index outside the activation rows reads nothing (its row is
        // not written either)
        if (rowa < 0 || rowa >= args.a_rows) {
          rowa = 0;
          aok[p] = false;
        }
        if (rowc < 0 || rowc >= args.a_rows) {
          rowc = 0;
          sok[p] = false;
        }
      }
      if (MODE == MODE_RUN) {
        ac[p] = lds_codes + rowa * cbytes;
        as[p] = lds_scales + rowc * sbytes;
      } else {
        ac[p] = args.a_codes + rowa * cbytes;
        as[p] = args.a_scales + rowc * sbytes;
      }
    }

    float acc[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) acc[p] = 0.f;

    while (cg * S < nsc) {  // wave-uniform
#pragma unroll
      for (int p = 0; p < MP; ++p) {
        if (r0 + 2 * p >= r_end) break;  // uniform
        uint4 a0[S], a1[S];
        uint2 sa[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int c = cg * S + s;
          const bool ok = c < nsc;
          const int64_t boff = (int64_t)c * 128 + 32 * j;
          const int64_t soff = (int64_t)c * 16 + 8 * (j & 1);
          if (MODE == MODE_RUN) {  // LDS, K % 256 == 0
            if (aok[p] && ok) {
              a0[s] = *(const uint4*)(ac[p] + boff);
              a1[s] = *(const uint4*)(ac[p] + boff + 16);
            } else {
              a0[s] = a1[s] = make_uint4(0u, 0u, 0u, 0u);
            }
            sa[s] = (sok[p] && ok) ? *(const uint2*)(as[p] + soff) : make_uint2(0u, 0u);
          } else {
            load32<FAST>(ac[p], boff, cbytes, aok[p] && ok, a0[s], a1[s]);
            sa[s] = load8<FAST>(as[p], soff, sbytes, sok[p] && ok);
          }
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
          if (cg * S + s >= nsc) break;  // wave-uniform: past the last chunk
          const v8i A0 = a_half == 0 ? v8i{(int)a0[s].x, (int)a0[s].y, 0, 0, 0, 0, 0, 0}
                                     : v8i{0, 0, (int)a0[s].z, (int)a0[s].w, 0, 0, 0, 0};
          const v8i A1 = a_half == 0 ? v8i{(int)a1[s].x, (int)a1[s].y, 0, 0, 0, 0, 0, 0}
                                     : v8i{0, 0, (int)a1[s].z, (int)a1[s].w, 0, 0, 0, 0};
          const v8i B0 = {(int)wb0[s].x, (int)wb0[s].y, (int)wb0[s].z, (int)wb0[s].w, 0, 0, 0, 0};
          const v8i B1 = {(int)wb1[s].x, (int)wb1[s].y, (int)wb1[s].z, (int)wb1[s].w, 0, 0, 0, 0};
          float fa[8], fw[8];
          fp8x8_to_f32(sa[s], fa);
          fp8x8_to_f32(wsb[s], fw);
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
      cg += NW;
      if (cg * S < nsc) load_w_group<S, FAST>(wrow, wsrow, cg, nsc, j, cbytes, sbytes, wb0, wb1, wsb);
    }

    // lanes of slices j and j^1 hold the same (row, column): add them
#pragma unroll
    for (int p = 0; p < MP; ++p) {
      acc[p] += __shfl_xor(acc[p], 16, 64);
      if ((j & 1) == 0) red[wave][2 * p + c_mloc][col] = acc[p];
    }
    __syncthreads();
    // ROWS*16 outputs; the workgroup may have fewer threads (one wave for short K)
    for (int e = threadIdx.x; e < ROWS * 16; e += blockDim.x) {
      const int rl = e >> 4, cc = e & 15;
      float s = 0.f;
      for (int w = 0; w < NW; ++w) s += red[w][rl][cc];
      const int r = r0 + rl, n = n0 + cc;
      bool ok = r < r_end && n < N;
      if (MODE == MODE_GROUPED && args.row_index != nullptr && ok)
        ok = args.row_index[r] >= 0 && args.row_index[r] < args.a_rows;
      if (ok) {
        const float v = s * (args.gsa_rows ? args.gsa[r] * args.ws2[g] : gscale);
        if (ROUTER)
          store_logit(args, (int64_t)r * N + n, v);
        else if (args.y_bf16)
          ((uint16_t*)args.y)[(int64_t)r * N + n] = (uint16_t)f32_to_bf16_rne(v);
        else
          ((float*)args.y)[(int64_t)r * N + n] = v;
      }
    }
    __syncthreads();
  }
  if constexpr (ROUTER) router_finish(args);
}

// ---------------------------------------------------------------- ring
// Many independent (group, 16 weight rows) tiles -- the routed-expert
// projections.  Every wave owns the whole K range of its 16 weight rows, so
// no partial sums cross waves.  The W waves of a workgroup take consecutive
// tiles of one group and share its activation rows, 2 * MP per pass, which
// the workgroup copies into LDS with direct global -> LDS loads once per
// pass.  The weight stream goes through LDS as well: an HBM read in which
// every load instruction covers whole 128-byte lines of 8 rows runs about a
// fifth faster than one covering half lines of 16 rows, which is what
// loading a 16-row MFMA operand straight into registers amounts to.  Each
// wave owns a private ring of D slots of one super-chunk (16 rows x 128
// bytes), each filled by two direct global -> LDS loads, and copies all of
// its tile's weight scales into LDS once.  Piece p of a row r sits at slot
// p ^ (r & 7), so the MFMA-layout reads of eight rows hit eight bank groups.
// The wave waits for a slot with an explicit vmcnt (no other vector memory
// instruction is issued inside its loop) and refills it after computing it.
constexpr int RING_SLOT = 16 * 128;  // bytes of one super-chunk of 16 rows

// wait until at most n vector memory instructions of this wave are in flight
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: __asm__ volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: __asm__ volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: __asm__ volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: __asm__ volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: __asm__ volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: __asm__ volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: __asm__ volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: __asm__ volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: __asm__ volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: __asm__ volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: __asm__ volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    default: __asm__ volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
  }
}

// ---- a ring workgroup that quantizes its own activation rows (RING_Q_X,
// RING_Q_PARTS).  The amax is still a grid-wide maximum reached without any
// workgroup waiting on another: with RING_Q_X every workgroup reduces all of
// the (small) x itself; with RING_Q_PARTS it reduces the partial maxima that
// an earlier launch wrote, which stream order completes first.

// gsa for every thread; partial maxima are bits of non-negative floats in the
// format of x (bf16 or fp32).  Ends with a workgroup barrier.
template <int QIN, bool XBF16, int W>
__device__ __forceinline__ float ring_gsa(const GemvArgs& args) {
  __shared__ uint32_t qred[W];
  uint32_t m = 0;
  if (QIN == RING_Q_X) {
    m = thread_absmax<XBF16>(args.x, (int64_t)args.a_rows * args.K, threadIdx.x, W * 64);
  } else {
    for (int t = threadIdx.x; t < args.nparts_in; t += W * 64) m = max(m, args.parts_in[t]);
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) qred[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t mm = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) mm = max(mm, qred[w]);
  return gsa_from_bits<XBF16>(mm);
}

// Quantize half-blocks [0, nh) of rows whose half-block i lies in row
// src_of(i / hpr) of x, at position i % hpr (hpr = K / 8 half-blocks a row):
// put(i, row, hh, code word, scale byte) stores each one.  The loop runs a
// uniform number of trips so that every lane takes part in src_of's shuffle;
// half-blocks 2b and 2b+1 of a block sit in adjacent lanes (W * 64 and hpr
// are even).
// U trips at a time: all U loads are in flight before the first is used.
template <bool XBF16, int W, typename SrcOf, typename Put>
__device__ __forceinline__ void ring_quantize(const GemvArgs& args, int nh, float gsa,
                                              SrcOf src_of, Put put) {
  constexpr int U = 4;
  const int hpr = args.K / 8;
  const int trips = (nh + W * 64 - 1) / (W * 64);
  for (int it0 = 0; it0 < trips; it0 += U) {
    int rl[U], hh[U], src[U];
    bool ok[U];
    uint4 raw[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (int)threadIdx.x + (it0 + u) * W * 64;
      const bool in = it0 + u < trips && i < nh;
      rl[u] = in ? i / hpr : 0;
      hh[u] = in ? i - rl[u] * hpr : 0;
      src[u] = src_of(rl[u]);
      ok[u] = in && src[u] >= 0;
      load_half8_raw<XBF16>(args.x, ok[u] ? (int64_t)src[u] * hpr + hh[u] : 0, raw[u]);
    }
    float v[U][8], bm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unpack_half8<XBF16>(raw[u], v[u]);
      const uint32_t hb = ok[u] ? half_absmax8_bits(v[u]) : 0u;
      bm[u] = __uint_as_float(max(hb, dpp_u32<DPP_XOR1>(hb)));
    }
    uint32_t c[U], sf[U];
    quantize_halves<U>(v, bm, gsa, c, sf);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) put(rl[u], src[u], hh[u], c[u], sf[u]);
  }
}

// Workgroup (0, 0)'s extra duty: gsa to gsa_out and, with RING_Q_X, every
// row of x quantized to codes_out / scales_out (when given).
template <int QIN, bool XBF16, int W>
__device__ __forceinline__ void ring_write_x(const GemvArgs& args, float gsa) {
  if (threadIdx.x == 0 && args.gsa_out != nullptr) args.gsa_out[0] = gsa;
  if (QIN != RING_Q_X || args.codes_out == nullptr) return;
  const int64_t cbytes = args.K / 2, sbytes = args.K / 16;
  ring_quantize<XBF16, W>(
      args, args.a_rows * (args.K / 8), gsa, [](int rl) { return rl; },
      [&](int, int src, int hh, uint32_t c, uint32_t sf) {
        ((uint32_t*)(args.codes_out + src * cbytes))[hh] = c;
        if ((hh & 1) == 0) args.scales_out[src * sbytes + hh / 2] = (uint8_t)sf;
      });
}

// SWIGLU: the output columns are gate/up groups of args.gran columns
// interleaved (group q is gate when q is even, and gate group 2p pairs with
// up group 2p+1); instead of those columns the epilogue writes
// h = silu(gate) * up, (M, N/2) fp32 at args.y, column p*gran + i, and each
// workgroup writes the largest |h| it wrote to args.partials (the first
// phase of h's amax).  A wave's 16 columns hold whole pairs (gran divides 8):
// the up value of gate column c sits in lane c ^ gran.
// QIN: where the activation rows come from (RING_Q_*); XBF16: x's format
// when the workgroup quantizes them.
// KS > 1: KS consecutive waves share a tile of 16 rows, wave k streaming
// super-chunks [k nsc/KS, (k+1) nsc/KS) through its own ring; after the
// loop the partial sums are added in k order (through the now idle ring
// slots) and the first wave of the tile stores.  More waves stream at once
// for the same rows.  nsc % KS == 0.
template <int MP, int D, int W, bool SWIGLU = false, int QIN = RING_Q_CODES, bool XBF16 = true,
          int KS = 1>
__global__ __launch_bounds__(W * 64) void gemv_ring_kernel(const GemvArgs args) {
  static_assert(2 * (D - 1) <= 14, "wait_vm range");
  constexpr int ROWS = 2 * MP;
  constexpr int SLOT = RING_SLOT;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, j = lane >> 4;
  const int N = args.N, K = args.K;
  int g = blockIdx.y;
  if (args.offsets != nullptr && (int)gridDim.y < args.groups) {
    // compacted grid: the blockIdx.y-th group with rows (in group order)
    __shared__ int sel, wcnt[W];
    if (threadIdx.x == 0) sel = -1;
    int base = 0;  // groups with rows before this pass
    for (int t0 = 0; t0 < args.groups; t0 += W * 64) {
      const int t = t0 + (int)threadIdx.x;
      bool act = false;
      if (t < args.groups)
        act = min(args.offsets[t + 1], args.M) > max(args.offsets[t], 0);
      const uint64_t b = __ballot(act);
      if (lane == 0) wcnt[wave] = __popcll(b);
      __syncthreads();
      int before = base;
      for (int w = 0; w < wave; ++w) before += wcnt[w];
      const int rank = before + __popcll(b & ((1ull << lane) - 1ull));
      if (act && rank == (int)blockIdx.y) sel = t;
      for (int w = 0; w < W; ++w) base += wcnt[w];
      __syncthreads();
    }
    g = __builtin_amdgcn_readfirstlane(sel);  // uniform after the barrier
    if (g < 0) {  // fewer groups with rows than workgroup rows
      if (SWIGLU && threadIdx.x == 0) args.partials[blockIdx.y * gridDim.x + blockIdx.x] = 0u;
      if (QIN != RING_Q_CODES && blockIdx.x == 0 && blockIdx.y == 0)
        ring_write_x<QIN, XBF16, W>(args, ring_gsa<QIN, XBF16, W>(args));
      return;
    }
  }
  int r_begin = 0, r_end = args.M;
  if (args.offsets != nullptr) {
    r_begin = max(args.offsets[g], 0);
    r_end = min(args.offsets[g + 1], args.M);
  }
  if (r_begin >= r_end) {  // uniform over the workgroup
    if (SWIGLU && threadIdx.x == 0) args.partials[blockIdx.y * gridDim.x + blockIdx.x] = 0u;
    if (QIN != RING_Q_CODES && blockIdx.x == 0 && blockIdx.y == 0)
      ring_write_x<QIN, XBF16, W>(args, ring_gsa<QIN, XBF16, W>(args));
    return;
  }
  float gsa_q = 0.f;  // QIN: the gsa this workgroup forms
  float hmax = 0.f;  // SWIGLU: largest |h| this thread wrote

  static_assert(W % KS == 0, "whole tiles per workgroup");
  const int kp = wave % KS;  // this wave's part of the K range
  const int n0 = (blockIdx.x * (W / KS) + wave / KS) * 16;
  const bool tile_ok = n0 < N;  // wave-uniform; a wave past the end only stages
  const int64_t cbytes = K / 2, sbytes = K / 16;
  const int nsc = K / 256;
  const int cb = kp * (nsc / KS), ce = cb + nsc / KS;  // this wave's super-chunks

  const int a_mloc = col >> 3, a_half = col & 1;
  const bool a_has = ((col & 7) >> 1) == j;
  const int c_mloc = j >> 1;

  // LDS: activation rows (codes, then scales), then per wave its weight
  // scales (16 rows x K/16 bytes) and its ring of D slots
  const uint32_t act_bytes = (uint32_t)(ROWS * (cbytes + sbytes));
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  const uint32_t wave_off = act_bytes + (uint32_t)wave * (uint32_t)(K + D * SLOT);
  const uint32_t ws_lds = lds0 + wave_off, ring_lds = ws_lds + (uint32_t)K;
  const uint8_t* lds_codes = lds;
  const uint8_t* lds_scales = lds + ROWS * cbytes;
  const uint8_t* ws_area = lds + wave_off;
  const uint8_t* ring = lds + wave_off + K;
  const int cpr = (int)(cbytes / 16), spr = (int)(sbytes / 16);  // 16-byte pieces per row

  // weight rows of the tile relative to row n0 (clamped: results discarded)
  const int64_t tile_row0 = (int64_t)g * N + (tile_ok ? n0 : 0);
  const uint8_t* wbase = args.w_codes + tile_row0 * cbytes;
  const uint8_t* wsbase = args.w_scales + tile_row0 * sbytes;
  // ring loads: lane l of load i takes row 8i + l/8, piece (l % 8) ^ (row % 8)
  uint32_t ring_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int rc = (tile_ok && n0 + r < N) ? r : max(N - 1 - n0, 0);
    ring_off[i] = (uint32_t)(rc * cbytes + 16 * ((lane & 7) ^ (r & 7)));
  }
  auto issue_slot = [&](int c) {
    const uint32_t slot = ring_lds + (uint32_t)(c % D) * SLOT;
    // nontemporal: a weight line is read once per pass of activation rows,
    // and decode-sized routing makes one pass
    load_lds16_nt(wbase, ring_off[0] + 128u * (uint32_t)c, slot);
    load_lds16_nt(wbase, ring_off[1] + 128u * (uint32_t)c, slot + 1024u);
  };

  for (int r0 = r_begin; r0 < r_end; r0 += ROWS) {
    int my_src = -1;
    if (lane < ROWS && r0 + lane < r_end) {
      my_src = args.row_index != nullptr ? args.row_index[r0 + lane] : r0 + lane;
      if (my_src < 0 || my_src >= args.a_rows) my_src = -1;
    }
    // fragment masks of the pass rows -- this first use of the row indices
    // also waits for their loads before any direct-to-LDS load is issued
    // (the compiler does not count those)
    bool aok[MP], sok[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) {
      const int srca = __shfl(my_src, 2 * p + a_mloc, 64);
      const int srcc = __shfl(my_src, 2 * p + c_mloc, 64);
      aok[p] = a_has && srca >= 0;
      sok[p] = srcc >= 0;
    }
    const int npairs = min(MP, (r_end - r0 + 1) / 2);
    __syncthreads();  // the previous pass has finished reading LDS

    if (tile_ok) {
      // the tile's weight scales (once, nontemporal: read once per call), then
      // the first D slots
      if (r0 == r_begin) {
        for (int e0 = 0; e0 < 16 * spr; e0 += 64) {
          const int e = e0 + lane;
          const int r = e / spr, q = e - r * spr;  // piece q: the scales of super-chunk q
          const int rc = (n0 + r < N) ? r : N - 1 - n0;
          if (e < 16 * spr && q >= cb && q < ce)
            load_lds16_nt(wsbase, (uint32_t)(rc * sbytes + 16 * q), ws_lds + 16u * (uint32_t)e0);
        }
      }
      for (int c = cb; c < cb + D && c < ce; ++c) issue_slot(c);
    }
    if (QIN == RING_Q_CODES) {
      // the pass rows' activation codes and scales (a missing row copies row
      // 0 and is masked below)
      const int ncp = ROWS * cpr, nsp = ROWS * spr;
      for (int base = wave * 64; base < ncp; base += W * 64) {
        const int e = base + lane;
        const int rl = e / cpr, q = e - rl * cpr;
        const int src = __shfl(my_src, rl < ROWS ? rl : 0, 64);
        if (e < ncp)
          load_lds16(args.a_codes, (uint32_t)((int64_t)max(src, 0) * cbytes + 16 * q),
                     lds0 + 16 * (uint32_t)base);
      }
      for (int base = wave * 64; base < nsp; base += W * 64) {
        const int e = base + lane;
        const int rl = e / spr, q = e - rl * spr;
        const int src = __shfl(my_src, rl < ROWS ? rl : 0, 64);
        if (e < nsp)
          load_lds16(args.a_scales, (uint32_t)((int64_t)max(src, 0) * sbytes + 16 * q),
                     lds0 + (uint32_t)(ROWS * cbytes) + 16 * (uint32_t)base);
      }
    } else {
      // the workgroup quantizes the pass rows itself, after the weight loads
      // above are on their way
      if (r0 == r_begin) {
        gsa_q = ring_gsa<QIN, XBF16, W>(args);
        if (blockIdx.x == 0 && blockIdx.y == 0) ring_write_x<QIN, XBF16, W>(args, gsa_q);
      }
      // with RING_Q_PARTS the first tile's workgroup of a group also stores
      // the codes of the rows it reads
      const bool out = QIN == RING_Q_PARTS && blockIdx.x == 0 && args.codes_out != nullptr;
      uint8_t* act = lds;
      ring_quantize<XBF16, W>(
          args, min(ROWS, r_end - r0) * (K / 8), gsa_q,
          [&](int rl) { return __shfl(my_src, rl, 64); },
          [&](int rl, int src, int hh, uint32_t c, uint32_t sf) {
            ((uint32_t*)(act + rl * cbytes))[hh] = c;
            if ((hh & 1) == 0) act[ROWS * cbytes + rl * sbytes + hh / 2] = (uint8_t)sf;
            if (out) {
              ((uint32_t*)(args.codes_out + src * cbytes))[hh] = c;
              if ((hh & 1) == 0) args.scales_out[src * sbytes + hh / 2] = (uint8_t)sf;
            }
          });
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();


    float acc[MP];
#pragma unroll
    for (int p = 0; p < MP; ++p) acc[p] = 0.f;

    if (tile_ok) {
      for (int c = cb; c < ce; ++c) {
        // slots c + 1 .. c + D - 1 may still be in flight
        wait_vm(2 * min(D - 1, ce - 1 - c));
        const uint8_t* sl = ring + (c % D) * SLOT + col * 128;
        const uint4 w0 = *(const uint4*)(sl + 16 * ((2 * j) ^ (col & 7)));
        const uint4 w1 = *(const uint4*)(sl + 16 * ((2 * j + 1) ^ (col & 7)));
        const uint2 wsc = *(const uint2*)(ws_area + col * sbytes + (int64_t)c * 16 + 8 * (j & 1));
        float fw[8];
        fp8x8_to_f32(wsc, fw);
        const v8i B0 = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, 0, 0, 0, 0};
        const v8i B1 = {(int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w, 0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < MP; ++p) {
          if (p >= npairs) break;  // uniform
          const uint8_t* ac = lds_codes + (2 * p + a_mloc) * cbytes + (int64_t)c * 128 + 32 * j +
                              8 * a_half;
          uint2 q0 = make_uint2(0u, 0u), q1 = make_uint2(0u, 0u), sa = make_uint2(0u, 0u);
          if (aok[p]) {
            q0 = *(const uint2*)ac;
            q1 = *(const uint2*)(ac + 16);
          }
          if (sok[p])
            sa = *(const uint2*)(lds_scales + (2 * p + c_mloc) * sbytes + (int64_t)c * 16 +
                                 8 * (j & 1));
          const v8i A0 = a_half == 0 ? v8i{(int)q0.x, (int)q0.y, 0, 0, 0, 0, 0, 0}
                                     : v8i{0, 0, (int)q0.x, (int)q0.y, 0, 0, 0, 0};
          const v8i A1 = a_half == 0 ? v8i{(int)q1.x, (int)q1.y, 0, 0, 0, 0, 0, 0}
                                     : v8i{0, 0, (int)q1.x, (int)q1.y, 0, 0, 0, 0};
          float fa[8];
          fp8x8_to_f32(sa, fa);
          const float4_t c0 = mfma_fp4(A0, B0);
          const float4_t c1 = mfma_fp4(A1, B1);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t0 = 4 * (r >> 1) + (r & 1);
            const int t1 = t0 + 2;
            acc[p] = fmaf(c0[r], fa[t0] * fw[t0], acc[p]);
            acc[p] = fmaf(c1[r], fa[t1] * fw[t1], acc[p]);
          }
        }
        // refill this slot once its reads have returned
        if (c + D < ce) {
          __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          issue_slot(c + D);
        }
      }
    }
    if constexpr (KS > 1) {
      // the tile's partial sums, in k order, through the waves' idle slots
      float* xch = (float*)(lds + wave_off + K);
      if (tile_ok && kp != 0) {
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // last slot reads done
#pragma unroll
        for (int p = 0; p < MP; ++p) xch[p * 64 + lane] = acc[p];
      }
      __syncthreads();
      if (tile_ok && kp == 0) {
#pragma unroll
        for (int k = 1; k < KS; ++k) {
          const float* px = (const float*)(lds + wave_off + (uint32_t)k * (uint32_t)(K + D * SLOT) + K);
#pragma unroll
          for (int p = 0; p < MP; ++p) acc[p] += px[p * 64 + lane];
        }
      }
    }
    if (tile_ok && kp == 0) {
      const float gscale = (QIN == RING_Q_CODES ? args.gsa[0] : gsa_q) * args.ws2[g];
#pragma unroll
      for (int p = 0; p < MP; ++p) {
        const float v = acc[p] + __shfl_xor(acc[p], 16, 64);
        const int rl = 2 * p + c_mloc, r = r0 + rl, n = n0 + col;
        // every lane takes part in the shuffle: a lane left out of it (its
        // column past N) would hand its readers an undefined row index
        const int rsrc = __shfl(my_src, rl, 64);
        const bool ok = (j & 1) == 0 && r < r_end && n < N && rsrc >= 0;
        if (SWIGLU) {
          const float gv = v * gscale;
          const float uv = __shfl_xor(gv, args.gran, 64);  // the paired up column
          if (ok && (col & args.gran) == 0) {  // a gate column (gran is a power of two)
            const float hv = swiglu1(gv, uv, args.limit);
            const int lg = __builtin_ctz(args.gran);
            const int hcol = ((n >> (lg + 1)) << lg) + (n & (args.gran - 1));
            ((float*)args.y)[(int64_t)r * (N / 2) + hcol] = hv;
            hmax = fmaxf(hmax, fabsf(hv));
          }
        } else if (ok) {
          // one gsa per row (one group of all rows, codes given)
          const float sc = args.gsa_rows ? args.gsa[r] * args.ws2[g] : gscale;
          if (args.y_bf16)
            ((uint16_t*)args.y)[(int64_t)r * N + n] = (uint16_t)f32_to_bf16_rne(v * sc);
          else
            ((float*)args.y)[(int64_t)r * N + n] = v * sc;
        }
      }
    }
  }
  if (SWIGLU) {  // the workgroup's largest |h|
    __shared__ uint32_t wmax[W];
    const uint32_t m = wave_max_u32(__float_as_uint(hmax));
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mm = 0;
      for (int w = 0; w < W; ++w) mm = max(mm, wmax[w]);
      args.partials[blockIdx.y * gridDim.x + blockIdx.x] = mm;
    }
  }
}

// Dynamic LDS the ring kernel may take (the rest is its static LDS).
constexpr size_t RING_MAX_LDS = 160 * 1024 - 256;

template <int MP, int D, int W>
static size_t ring_lds_bytes(int64_t K) {
  return (size_t)(2 * MP) * (size_t)(K / 2 + K / 16) +
         (size_t)W * (size_t)(K + D * RING_SLOT);
}

template <int MP, int D, int W, bool SWIGLU, int QIN = RING_Q_CODES, bool XBF16 = true,
          int KS = 1>
static hipError_t launch_ring_t(const GemvArgs& a, int G, hipStream_t s) {
  const size_t lds = ring_lds_bytes<MP, D, W>(a.K);
  if (lds > 64 * 1024) {  // the largest any launch may ask for (callers keep lds below it)
    static unsigned char done[64];
    const hipError_t e = allow_dynamic_lds(
        (const void*)gemv_ring_kernel<MP, D, W, SWIGLU, QIN, XBF16, KS>, RING_MAX_LDS, done);
    if (e != hipSuccess) return e;
  }
  // at most M groups have rows: with fewer rows than groups, launch a row of
  // workgroups per possible group with rows instead of one per group
  GemvArgs b = a;
  b.groups = G;
  const int gy = (a.offsets != nullptr && a.M < G) ? (a.M > 0 ? a.M : 1) : G;
  constexpr int TW = W / KS;  // tiles of 16 rows per workgroup
  const dim3 grid((unsigned)((a.N + 16 * TW - 1) / (16 * TW)), (unsigned)gy);
  gemv_ring_kernel<MP, D, W, SWIGLU, QIN, XBF16, KS><<<grid, W * 64, lds, s>>>(b);
  return hipGetLastError();
}

// ---------------------------------------------------------------- narrow
// Few activation rows and few weight rows per workgroup: RQ quads of 4
// weight rows per workgroup (8 rows at decode sizes) so that a decode-sized
// N spreads its weight stream over every CU.  The K dimension is split four
// ways inside each MFMA: B column n' = 4q + r holds weight row r at chunk 4*set + q (a "stream" q of 128
// K-elements), A row i = 4q + t holds activation block 4h + t of the same
// chunk in MFMA h (two MFMAs cover the chunk's 8 blocks), so result row
// 4q + t against column 4q + r is the exact block sum S_b for row r; the
// other 3/4 of the results are cross terms and are discarded (their scale
// factor is 0).  Result lane l holds rows 4*(l/16) + t, t = 0..3, of column
// l % 16: it is useful when l/16 == (l%16)/4, i.e. l = 20q + r.  A
// 512-element set is 256 contiguous bytes per weight row.
//
// Every lane loads what its MFMAs and scale products need straight into
// registers -- 16 weight-code bytes, the 8 weight-scale bytes of its
// (row, chunk) and, for already quantized activations, 16 code bytes and 8
// scale bytes -- for S sets at a time, the next group's loads in flight
// while the current one computes.  No staging, no barrier before compute.
// RUN: the workgroup quantizes the whole (small) activation itself -- amax
// over every element, gsa, codes and scales into LDS, HPT half-blocks per
// thread -- while its weight loads are in flight.  No workgroup depends on
// another; workgroup 0 also writes gsa, codes and scales out.
template <int S, int MR, bool RUN, bool XBF16, int HPT, int RQ, int MAXW, bool ROUTER = false>
__global__ __launch_bounds__(MAXW * 64) void gemv_narrow_kernel(const GemvArgs args) {
  __shared__ float red[MAXW][MR][4 * RQ];
  __shared__ float amax_red[MAXW];
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // RUN: codes, scales
  const int NW = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, j = lane >> 4;
  const int M = args.M, N = args.N, K = args.K;
  const int n0 = blockIdx.x * 4 * RQ;  // RQ quads of 4 weight rows
  const int q = col >> 2, r = col & 3;  // B column: stream, weight row; A row: stream, slot
  const bool useful = j == q;           // result rows of this lane are stream j
  const int64_t cbytes = K / 2, sbytes = K / 16;
  const int nset = K / 512;
  const uint8_t* wrow[RQ];
  const uint8_t* wsrow[RQ];
#pragma unroll
  for (int rq = 0; rq < RQ; ++rq) {
    const int64_t wr = min(n0 + 4 * rq + r, N - 1);  // clamped: missing rows are not stored
    wrow[rq] = args.w_codes + wr * cbytes;
    wsrow[rq] = args.w_scales + wr * sbytes;
  }
  // A row slot t = r carries block 4h + t of its chunk in MFMA h: slice 2h + t/2
  const int dj = j - (r >> 1);
  const bool a_has = dj == 0 || dj == 2;
  const int a_h = dj >> 1, a_half = r & 1;
  uint8_t* acl = lds;                       // [M][cbytes]
  uint8_t* asl = lds + (int64_t)M * cbytes;  // [M][sbytes]

  // activation rows (clamped; mok masks the missing ones)
  bool mok[MR];
  const uint8_t* arc[MR];
  const uint8_t* ars[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    mok[m] = m < M;
    const int64_t ar = mok[m] ? m : 0;
    arc[m] = (RUN ? acl : args.a_codes) + ar * cbytes;
    ars[m] = (RUN ? asl : args.a_scales) + ar * sbytes;
  }

  const int64_t nhalf = (int64_t)M * (K / 8);
  // One activation row with one set group per wave (HPT == S, NW * S sets
  // cover the row): lane l of wave w quantizes half-block l of sets S w ..
  // S w + S - 1 -- exactly the sets the wave multiplies, so the wave needs
  // no other wave's codes.  Otherwise half-blocks go round the workgroup.
  const bool own_sets = RUN && M == 1 && HPT == S && NW * S >= nset;
  auto half_of = [&](int u) -> int64_t {
    return own_sets ? (int64_t)(lane + 64 * (S * wave + u))
                    : (int64_t)threadIdx.x + (int64_t)u * blockDim.x;
  };
  uint4 xr[HPT][2];
  bool xok[HPT];
  if (RUN) {  // the activation first: its loads complete before the weights'
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
      const int64_t h = half_of(u);
      xok[u] = h < nhalf;
      load_half8_raw<XBF16>(args.x, xok[u] ? h : 0, xr[u]);
    }
  }

  // Every wave's activation loads enter the memory pipeline before any
  // weight load: the activation's amax and quantize are the critical path.
  if (RUN) __builtin_amdgcn_s_barrier();

  int sg = wave;
  uint4 wv[S][RQ];
  uint2 fwv[S][RQ];
  uint4 av[S][MR];
  uint2 sav[S][MR];
  auto load_group = [&](int gg) {
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {  // unconditional loads of clamped sets
      const int set = min(gg * S + s2, nset - 1);
#pragma unroll
      for (int rq = 0; rq < RQ; ++rq) {
        wv[s2][rq] = ldg_nt16(wrow[rq] + (int64_t)(4 * set + q) * 64 + 16 * j);
        fwv[s2][rq] = ldg_nt8(wsrow[rq] + (4 * set + j) * 8);
      }
      if (!RUN) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          av[s2][m] = *(const uint4*)(arc[m] + (int64_t)(4 * set + q) * 64 + 16 * j);
          sav[s2][m] = *(const uint2*)(ars[m] + (4 * set + j) * 8);
        }
      }
    }
  };
  load_group(sg);
  // all weight loads are issued before the activation is first used
  if (RUN) __builtin_amdgcn_sched_barrier(0);

  float gsa_v = RUN ? 0.f : args.gsa[0];
  if (RUN) {  // quantize the activation into LDS
    float xv[HPT][8];
#pragma unroll
    for (int u = 0; u < HPT; ++u) unpack_half8<XBF16>(xr[u], xv[u]);
    uint32_t hb[HPT], mx = 0;  // |x| maxima as float bits
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
      hb[u] = xok[u] ? half_absmax8_bits(xv[u]) : 0u;
      mx = max(mx, hb[u]);
    }
    mx = wave_max_u32(mx);
    if (lane == 0) amax_red[wave] = __uint_as_float(mx);
    lds_barrier();
    // every row of 16 lanes reads the (at most 16) wave maxima at once
    const uint32_t mm = row16_max_u32((lane & 15) < NW ? __float_as_uint(amax_red[lane & 15]) : 0u);
    gsa_v = gsa_from_amax(__uint_as_float(mm));
    const bool writer = blockIdx.x == 0;
    float bm[HPT];
#pragma unroll
    for (int u = 0; u < HPT; ++u) bm[u] = __uint_as_float(max(hb[u], dpp_u32<DPP_XOR1>(hb[u])));
    uint32_t cw[HPT], sfw[HPT];
    quantize_halves<HPT>(xv, bm, gsa_v, cw, sfw);
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
      const int64_t h = half_of(u);
      const uint32_t c = cw[u], sf = sfw[u];
      if (xok[u]) {
        ((uint32_t*)acl)[h] = c;
        if ((h & 1) == 0) asl[h >> 1] = (uint8_t)sf;
        if (writer) {
          ((uint32_t*)args.codes_out)[h] = c;
          if ((h & 1) == 0) args.scales_out[h >> 1] = (uint8_t)sf;
        }
      }
    }
    if (writer && threadIdx.x == 0) args.gsa_out[0] = gsa_v;
    // With own_sets a wave quantized exactly the sets it multiplies and a
    // wave's LDS operations complete in order: no other wave is waited for.
    if (!own_sets) lds_barrier();
  }

  float acc[MR][RQ];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int rq = 0; rq < RQ; ++rq) acc[m][rq] = 0.f;
  while (sg * S < nset) {  // wave-uniform
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
      const int set = sg * S + s2;
      if (set >= nset) break;  // wave-uniform
      float fw[RQ][8];
#pragma unroll
      for (int rq = 0; rq < RQ; ++rq) fp8x8_to_f32(fwv[s2][rq], fw[rq]);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m >= M) break;  // uniform
        uint4 a4;
        uint2 sa;
        if (RUN) {
          a4 = *(const uint4*)(arc[m] + (int64_t)(4 * set + q) * 64 + 16 * j);
          sa = *(const uint2*)(ars[m] + (4 * set + j) * 8);
        } else {
          a4 = av[s2][m];
          sa = sav[s2][m];
        }
        a4 = a_has ? a4 : make_uint4(0u, 0u, 0u, 0u);
        sa = useful ? sa : make_uint2(0u, 0u);
        const v8i Am = a_half == 0 ? v8i{(int)a4.x, (int)a4.y, 0, 0, 0, 0, 0, 0}
                                   : v8i{0, 0, (int)a4.z, (int)a4.w, 0, 0, 0, 0};
        const v8i Z = {0, 0, 0, 0, 0, 0, 0, 0};
        const v8i A0 = a_h == 0 ? Am : Z, A1 = a_h == 1 ? Am : Z;
        float fa[8];
        fp8x8_to_f32(sa, fa);
#pragma unroll
        for (int rq = 0; rq < RQ; ++rq) {
          const v8i B = {(int)wv[s2][rq].x, (int)wv[s2][rq].y, (int)wv[s2][rq].z,
                         (int)wv[s2][rq].w, 0, 0, 0, 0};
          const float4_t c0 = mfma_fp4(A0, B);
          const float4_t c1 = mfma_fp4(A1, B);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc[m][rq] = fmaf(c0[t], fa[t] * fw[rq][t], acc[m][rq]);
            acc[m][rq] = fmaf(c1[t], fa[4 + t] * fw[rq][4 + t], acc[m][rq]);
          }
        }
      }
    }
    sg += NW;
    if (sg * S < nset) load_group(sg);
  }
  // row r's partial sums sit in lanes 20q + r: gather them in lanes 0..3
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int rq = 0; rq < RQ; ++rq) {
      const float v = useful ? acc[m][rq] : 0.f;
      const int src = 20 * (lane >> 2) + (lane & 3);  // lanes 0..15 read the 16 useful lanes
      float t = __shfl(v, src & 63, 64);
      // lanes r, r+4, r+8, r+12 of row 0 hold row r's four parts: two
      // rotations by 4 and 8 lanes add them (either direction covers them)
      t += dpp_f32<DPP_ROR4>(t);
      t += dpp_f32<DPP_ROR8>(t);
      if (lane < 4) red[wave][m][4 * rq + lane] = t;
    }
  __syncthreads();
  // output o = e / 16 is summed by 16 lanes at once, lane e % 16 reading the
  // partial of wave e % 16 (at most 16 waves)
  const float gscale = gsa_v * args.ws2[0];
  for (int base = threadIdx.x & ~63; base < 16 * MR * 4 * RQ; base += blockDim.x) {
    const int e = base + lane, o = e >> 4, w = e & 15;
    const int m = o / (4 * RQ), rr = o % (4 * RQ);
    float sum = (w < NW && o < MR * 4 * RQ) ? red[w][m][rr] : 0.f;
    sum = row16_sum_f32(sum);
    const int n = n0 + rr;
    if (w == 0 && o < MR * 4 * RQ && m < M && n < N) {
      const float v = sum * (args.gsa_rows ? args.gsa[m] * args.ws2[0] : gscale);
      if (ROUTER)
        store_logit(args, (int64_t)m * N + n, v);
      else if (args.y_bf16)
        ((uint16_t*)args.y)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v);
      else
        ((float*)args.y)[(int64_t)m * N + n] = v;
    }
  }
  if constexpr (ROUTER) router_finish(args);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int S_GROUP = 4;

static int waves_for(int64_t K, int S = S_GROUP) {
  const int64_t nsc = (K + 255) / 256;
  int64_t nw = (nsc + S - 1) / S;
  if (nw < 1) nw = 1;
  if (nw > GEMV_MAX_WAVES) nw = GEMV_MAX_WAVES;
  return (int)nw;
}

template <int MP, int MODE, int S = S_GROUP, bool ROUTER = false>
static hipError_t launch_mp(const GemvArgs& a, bool fast, dim3 grid, int nw, hipStream_t s) {
  if (fast)
    gemv_fp4_kernel<S, MP, true, MODE, true, 1, ROUTER><<<grid, nw * 64, 0, s>>>(a);
  else
    gemv_fp4_kernel<S, MP, false, MODE, true, 1, ROUTER><<<grid, nw * 64, 0, s>>>(a);
  return hipGetLastError();
}

// Grouped linear through the LDS ring with one configuration, if its LDS
// fits RING_MAX_LDS (false: K too long to stage).  *parts: the grid's
// workgroup count (SwiGLU amax partials).
template <int MP, int D, int W, bool SWIGLU, int QIN = RING_Q_CODES, bool XBF16 = true,
          int KS = 1>
static bool ring_try(const GemvArgs& a, int G, hipStream_t s, hipError_t* err, int64_t* parts) {
  if (ring_lds_bytes<MP, D, W>(a.K) > RING_MAX_LDS) return false;
  if ((a.K / 256) % KS != 0) return false;
  const int64_t gy = (a.offsets != nullptr && a.M < G) ? (a.M > 0 ? a.M : 1) : G;
  constexpr int TW = W / KS;
  *parts = (int64_t)((a.N + 16 * TW - 1) / (16 * TW)) * gy;
  *err = launch_ring_t<MP, D, W, SWIGLU, QIN, XBF16, KS>(a, G, s);
  return true;
}

// Decode-sized groups on a grid that 128-row tiles do not fill: two waves
// share each 16-row tile, splitting its K range (twice the waves streaming
// at once).  The same rule in both launchers keeps the self-quantizing
// ring's sums bit-identical to the codes ring's.
static bool ring_narrow_decode(const GemvArgs& a, int G, int64_t mean_rows) {
  const int64_t gy = (a.offsets != nullptr && a.M < G) ? (a.M > 0 ? a.M : 1) : G;
  return mean_rows <= 2 && ((a.N + 127) / 128) * gy < device_cu_count();
}

// The first configuration that fits: the K split above; then 16 activation
// rows a pass when groups average more than 4 rows, else 8 rows with 8 waves
// (one workgroup per CU), then smaller footprints for longer K.
template <bool SWIGLU>
static bool launch_ring(const GemvArgs& a, int G, int64_t mean_rows, hipStream_t s,
                        hipError_t* err, int64_t* parts) {
  if (ring_narrow_decode(a, G, mean_rows) &&
      ring_try<1, 4, 8, SWIGLU, RING_Q_CODES, true, 2>(a, G, s, err, parts))
    return true;
  if (mean_rows > 4 && ring_try<8, 3, 4, SWIGLU>(a, G, s, err, parts)) return true;
  return ring_try<4, 3, 8, SWIGLU>(a, G, s, err, parts) ||
         ring_try<4, 3, 4, SWIGLU>(a, G, s, err, parts) ||
         ring_try<2, 3, 4, SWIGLU>(a, G, s, err, parts) ||
         ring_try<1, 3, 2, SWIGLU>(a, G, s, err, parts);
}

// The ring with workgroups that quantize their own activation rows (QIN):
// eight waves of 16 weight rows a workgroup where that still gives a
// workgroup per CU, else two waves (four times the workgroups); two rows a
// pass for decode-sized groups, eight otherwise.
template <bool SWIGLU, int QIN, bool XBF16>
static bool launch_ring_q(const GemvArgs& a, int G, int64_t mean_rows, hipStream_t s,
                          hipError_t* err, int64_t* parts) {
  const int64_t gy = (a.offsets != nullptr && a.M < G) ? (a.M > 0 ? a.M : 1) : G;
  const bool wide = ((a.N + 127) / 128) * gy >= device_cu_count();
  if (mean_rows <= 2) {
    // eight waves a workgroup where 128-row tiles fill the chip; otherwise
    // eight waves on four tiles, two waves splitting each tile's K range,
    // with a 4-slot ring (one token over 8 x 1536 rows of K = 8192: 18.7 us,
    // against 23.7 us with four waves on four tiles and 28.6 us with two
    // waves and 3 slots; K split four ways: 26.0 us; the split on the
    // 128-row-tile grids: one token over 8 experts 45.5 -> 60.9 us)
    if (wide && ring_try<1, 3, 8, SWIGLU, QIN, XBF16>(a, G, s, err, parts)) return true;
    if (ring_narrow_decode(a, G, mean_rows) &&
        ring_try<1, 4, 8, SWIGLU, QIN, XBF16, 2>(a, G, s, err, parts))
      return true;
    if (ring_try<1, 4, 4, SWIGLU, QIN, XBF16>(a, G, s, err, parts)) return true;
    return ring_try<1, 3, 2, SWIGLU, QIN, XBF16>(a, G, s, err, parts);
  }
  if (wide && ring_try<4, 3, 8, SWIGLU, QIN, XBF16>(a, G, s, err, parts)) return true;
  return ring_try<4, 3, 2, SWIGLU, QIN, XBF16>(a, G, s, err, parts) ||
         ring_try<1, 3, 2, SWIGLU, QIN, XBF16>(a, G, s, err, parts);
}

bool grouped_run_supported(int64_t x_rows, int64_t K, const void* x, const uint8_t* w_codes,
                           const uint8_t* w_scales) {
  return K % 256 == 0 && K >= 256 && x_rows >= 1 && x_rows * (K / 2) < ((int64_t)1 << 31) &&
         aligned16(x) && aligned16(w_codes) && aligned16(w_scales) &&
         ring_lds_bytes<1, 3, 2>(K) <= RING_MAX_LDS;
}

hipError_t launch_grouped_run(const void* x, bool x_bf16, int64_t x_rows, const uint32_t* parts,
                              int64_t nparts, float* gsa_out, uint8_t* codes_out,
                              uint8_t* scales_out, const int32_t* row_index,
                              const int32_t* offsets, int G, int64_t M_total,
                              const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                              void* y, bool y_bf16, int64_t N, int64_t K, bool swiglu, int gran,
                              float limit, uint32_t* partials_out, int64_t* nparts_out,
                              hipStream_t s) {
  GemvArgs a{};
  a.x = x;
  a.parts_in = parts;
  a.nparts_in = (int)nparts;
  a.gsa_out = gsa_out;
  a.codes_out = codes_out;
  a.scales_out = scales_out;
  a.row_index = row_index;
  a.offsets = offsets;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.ws2 = ws2;
  a.y = y;
  a.y_bf16 = y_bf16 ? 1 : 0;
  a.M = (int)M_total;
  a.N = (int)N;
  a.K = (int)K;
  a.a_rows = (int)x_rows;
  a.gran = gran;
  a.limit = limit;
  a.partials = partials_out;
  const int64_t mean_rows = (M_total + G - 1) / G;
  hipError_t err = hipSuccess;
  int64_t np = 0;
  bool ok;
  if (parts != nullptr) {
    ok = x_bf16 ? (swiglu ? launch_ring_q<true, RING_Q_PARTS, true>(a, G, mean_rows, s, &err, &np)
                          : launch_ring_q<false, RING_Q_PARTS, true>(a, G, mean_rows, s, &err, &np))
                : (swiglu ? launch_ring_q<true, RING_Q_PARTS, false>(a, G, mean_rows, s, &err, &np)
                          : launch_ring_q<false, RING_Q_PARTS, false>(a, G, mean_rows, s, &err, &np));
  } else {
    ok = x_bf16 ? (swiglu ? launch_ring_q<true, RING_Q_X, true>(a, G, mean_rows, s, &err, &np)
                          : launch_ring_q<false, RING_Q_X, true>(a, G, mean_rows, s, &err, &np))
                : (swiglu ? launch_ring_q<true, RING_Q_X, false>(a, G, mean_rows, s, &err, &np)
                          : launch_ring_q<false, RING_Q_X, false>(a, G, mean_rows, s, &err, &np));
  }
  if (nparts_out) *nparts_out = np;
  return ok ? err : hipErrorInvalidValue;
}

// Most workgroups any ring configuration launches for (N, G): the size of
// the SwiGLU amax partials.
int64_t ring_max_parts(int64_t N, int G) { return ((N + 31) / 32) * (int64_t)G; }

template <int MODE, bool ROUTER = false>
static hipError_t launch_rows(const GemvArgs& a, int64_t rows_per_pass, bool fast, dim3 grid,
                              int nw, hipStream_t s) {
  if (rows_per_pass <= 2) return launch_mp<1, MODE, S_GROUP, ROUTER>(a, fast, grid, nw, s);
  if (rows_per_pass <= 4) return launch_mp<2, MODE, S_GROUP, ROUTER>(a, fast, grid, nw, s);
  return launch_mp<8, MODE, S_GROUP, ROUTER>(a, fast, grid, nw, s);
}

// One activation row: one 512-element set per wave and up to 16 waves (the
// quantize in RUN mode spreads over more threads); more rows: two sets per
// wave and up to 8 waves (their registers do not fit 16 waves).
constexpr int NARROW_MAXW1 = 16;

static int narrow_waves(int64_t K, int S, int maxw) {
  const int64_t nset = K / 512;
  int64_t nw = (nset + S - 1) / S;
  return (int)(nw < 1 ? 1 : (nw > maxw ? maxw : nw));
}

// 8 weight rows (two quads) per workgroup: half as many workgroups quantize
// the activation in RUN mode, and a decode-sized N still spreads over the CUs
constexpr int NARROW_RQ = 2;

template <bool ROUTER = false>
static hipError_t launch_narrow(const GemvArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.N + 4 * NARROW_RQ - 1) / (4 * NARROW_RQ)));
  if (a.M <= 1) {
    const int th = narrow_waves(a.K, 1, NARROW_MAXW1) * 64;
    // few weight rows (a router gate): one quad a workgroup, so twice as
    // many CUs stream them
    if ((int)grid.x < 128) {
      gemv_narrow_kernel<1, 1, false, true, 1, 1, NARROW_MAXW1, ROUTER>
          <<<dim3((unsigned)((a.N + 3) / 4)), th, 0, s>>>(a);
      return hipGetLastError();
    }
    gemv_narrow_kernel<1, 1, false, true, 1, NARROW_RQ, NARROW_MAXW1, ROUTER>
        <<<grid, th, 0, s>>>(a);
  } else {
    const int th = narrow_waves(a.K, 2, GEMV_MAX_WAVES) * 64;
    if (a.M <= 2)
      gemv_narrow_kernel<2, 2, false, true, 1, NARROW_RQ, GEMV_MAX_WAVES, ROUTER>
          <<<grid, th, 0, s>>>(a);
    else
      gemv_narrow_kernel<2, 4, false, true, 1, NARROW_RQ, GEMV_MAX_WAVES, ROUTER>
          <<<grid, th, 0, s>>>(a);
  }
  return hipGetLastError();
}

bool gemv_narrow_supported(int64_t M, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales) {
  return M >= 1 && M <= 4 && K % 512 == 0 && K <= 16384 && aligned16(a_codes) &&
         aligned16(a_scales) && aligned16(w_codes) && aligned16(w_scales);
}

// RUN mode: enough threads for at most 4 activation half-blocks each.
bool gemv_narrow_run_supported(int64_t M, int64_t K, const void* x, const uint8_t* w_codes,
                               const uint8_t* w_scales) {
  return M >= 1 && M <= 4 && K % 512 == 0 && K <= 16384 &&
         M * (K / 8) <= 4 * GEMV_MAX_WAVES * 64 && aligned16(x) && aligned16(w_codes) &&
         aligned16(w_scales);
}

template <int S, int MR, bool XBF16, int MAXW>
static hipError_t launch_narrow_run_t(const GemvArgs& a, int nw, int hpt, size_t lds,
                                      hipStream_t s) {
  dim3 grid((unsigned)((a.N + 4 * NARROW_RQ - 1) / (4 * NARROW_RQ)));
  if (hpt == 1)
    gemv_narrow_kernel<S, MR, true, XBF16, 1, NARROW_RQ, MAXW><<<grid, nw * 64, lds, s>>>(a);
  else if (hpt == 2)
    gemv_narrow_kernel<S, MR, true, XBF16, 2, NARROW_RQ, MAXW><<<grid, nw * 64, lds, s>>>(a);
  else
    gemv_narrow_kernel<S, MR, true, XBF16, 4, NARROW_RQ, MAXW><<<grid, nw * 64, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_narrow_run(const void* x, bool x_bf16, float* gsa, uint8_t* codes,
                             uint8_t* scales, const uint8_t* w_codes, const uint8_t* w_scales,
                             const float* ws2, void* y, bool y_bf16, int64_t M, int64_t N,
                             int64_t K, hipStream_t s) {
  GemvArgs a{};
  a.x = x;
  a.gsa_out = gsa;
  a.codes_out = codes;
  a.scales_out = scales;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.ws2 = ws2;
  a.y = y;
  a.y_bf16 = y_bf16 ? 1 : 0;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.a_rows = (int)M;
  const int64_t nhalf = M * (K / 8);
  const bool one = M <= 1;
  const size_t lds = (size_t)(M * (K / 2 + K / 16));
  if (one && K >= 1024) {
    // two 512-element sets per wave, each wave quantizing its own two:
    // half the waves of one set each, and no barrier after the quantize
    const int nw2 = narrow_waves(K, 2, NARROW_MAXW1);
    dim3 grid((unsigned)((a.N + 4 * NARROW_RQ - 1) / (4 * NARROW_RQ)));
    if (x_bf16)
      gemv_narrow_kernel<2, 1, true, true, 2, NARROW_RQ, NARROW_MAXW1>
          <<<grid, nw2 * 64, lds, s>>>(a);
    else
      gemv_narrow_kernel<2, 1, true, false, 2, NARROW_RQ, NARROW_MAXW1>
          <<<grid, nw2 * 64, lds, s>>>(a);
    return hipGetLastError();
  }
  const int maxw = one ? NARROW_MAXW1 : GEMV_MAX_WAVES;
  int nw = narrow_waves(K, one ? 1 : 2, maxw);
  while ((int64_t)nw * 64 * 4 < nhalf && nw < maxw) ++nw;
  const int64_t per = ((int64_t)nw * 64);
  const int hpt = nhalf <= per ? 1 : (nhalf <= 2 * per ? 2 : 4);
  if (x_bf16) {
    if (one) return launch_narrow_run_t<1, 1, true, NARROW_MAXW1>(a, nw, hpt, lds, s);
    if (M <= 2) return launch_narrow_run_t<2, 2, true, GEMV_MAX_WAVES>(a, nw, hpt, lds, s);
    return launch_narrow_run_t<2, 4, true, GEMV_MAX_WAVES>(a, nw, hpt, lds, s);
  }
  if (one) return launch_narrow_run_t<1, 1, false, NARROW_MAXW1>(a, nw, hpt, lds, s);
  if (M <= 2) return launch_narrow_run_t<2, 2, false, GEMV_MAX_WAVES>(a, nw, hpt, lds, s);
  return launch_narrow_run_t<2, 4, false, GEMV_MAX_WAVES>(a, nw, hpt, lds, s);
}

hipError_t launch_gemv(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* ws2,
                       void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s,
                       bool gsa_rows, const RouterEpilogue* router) {
  GemvArgs a{};
  if (router != nullptr) {
    a.router_k = router->k;
    a.router_bias = router->bias;
    a.router_idx = router->idx;
    a.router_score = router->score;
    a.router_count = router->count;
  }
  a.gsa_rows = gsa_rows ? 1 : 0;
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.gsa = gsa;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.ws2 = ws2;
  a.y = y;
  a.y_bf16 = y_bf16 ? 1 : 0;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.a_rows = (int)M;
  const bool fast = (K % 256 == 0) && aligned16(a_codes) && aligned16(a_scales) &&
                    aligned16(w_codes) && aligned16(w_scales);
  dim3 grid((unsigned)((N + 15) / 16), 1u);
  if (router != nullptr) {
    if (gemv_narrow_supported(M, K, a_codes, a_scales, w_codes, w_scales))
      return launch_narrow<true>(a, s);
    return launch_rows<MODE_PLAIN, true>(a, M, fast, grid, waves_for(K), s);
  }
  if (gemv_ring_preferred(M, N) && fast && M * (K / 2) < ((int64_t)1 << 31)) {
    // the weight ring, all M rows one group
    hipError_t err = hipSuccess;
    int64_t parts = 0;
    if (launch_ring<false>(a, 1, M, s, &err, &parts)) return err;
  }
  // the staged tiles (32-bit weight offsets); no split K at these widths, so no workspace
  if (gemv_tiled_preferred(M, N) && fast && N * (K / 2) < ((int64_t)1 << 31))
    return launch_gemm(a_codes, a_scales, gsa, w_codes, w_scales, ws2, y, y_bf16, M, N, K, s,
                       gsa_rows);
  if (gemv_narrow_preferred(M, N) &&
      gemv_narrow_supported(M, K, a_codes, a_scales, w_codes, w_scales))
    return launch_narrow(a, s);
  return launch_rows<MODE_PLAIN>(a, M, fast, grid, waves_for(K), s);
}

hipError_t launch_grouped_gemv(const uint8_t* a_codes, const uint8_t* a_scales, const float* gsa,
                               int64_t a_rows, const int32_t* row_index, const int32_t* offsets,
                               int G, int64_t M_total, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* ws2, void* y, bool y_bf16,
                               int64_t N, int64_t K, hipStream_t s) {
  GemvArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.gsa = gsa;
  a.row_index = row_index;
  a.offsets = offsets;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.ws2 = ws2;
  a.y = y;
  a.y_bf16 = y_bf16 ? 1 : 0;
  a.M = (int)M_total;
  a.N = (int)N;
  a.K = (int)K;
  a.a_rows = (int)a_rows;
  const bool fast = (K % 256 == 0) && aligned16(a_codes) && aligned16(a_scales) &&
                    aligned16(w_codes) && aligned16(w_scales);
  // rows per pass from the mean group size (groups larger than a pass make
  // more passes over the same weight tile, which then comes from L2)
  const int64_t mean_rows = (M_total + G - 1) / G;
  // many rows per group: tiles on the matrix cores
  if (mean_rows >= GROUPED_MFMA_MIN_ROWS &&
      grouped_gemm_supported(a_codes, a_scales, w_codes, w_scales, a_rows, M_total, G, N, K))
    return launch_grouped_gemm(a_codes, a_scales, gsa, a_rows, row_index, offsets, G, M_total,
                               w_codes, w_scales, ws2, y, y_bf16, N, K, s);
  if (fast && a_rows * (K / 2) < ((int64_t)1 << 31)) {  // copy offsets are 32-bit
    hipError_t err = hipSuccess;
    int64_t parts = 0;
    if (launch_ring<false>(a, G, mean_rows, s, &err, &parts)) return err;
  }
  dim3 grid((unsigned)((N + 15) / 16), (unsigned)G);
  if (mean_rows <= 2 && K >= 4096) {
    // long K, few rows: two super-chunks per wave in flight instead of four
    // (109 instead of 157 registers, so two workgroups share a CU)
    return launch_mp<2, MODE_GROUPED, 2>(a, fast, grid, waves_for(K, 2), s);
  }
  return launch_rows<MODE_GROUPED>(a, mean_rows <= 2 ? 4 : 2 * mean_rows, fast, grid,
                                   waves_for(K), s);
}

int64_t grouped_swiglu_parts(int64_t N, int G) { return ring_max_parts(N, G); }

// Groups of many rows take the tiled kernel (as launch_grouped_gemv).
static bool swiglu_tiled(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                         const uint8_t* w_scales, int64_t a_rows, int64_t M_total, int G,
                         int64_t N, int64_t K) {
  return (M_total + G - 1) / G >= GROUPED_MFMA_MIN_ROWS &&
         grouped_gemm_supported(a_codes, a_scales, w_codes, w_scales, a_rows, M_total, G, N, K);
}

int64_t grouped_swiglu_parts_for(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const uint8_t* w_codes, const uint8_t* w_scales, int64_t a_rows,
                                 int64_t M_total, int G, int64_t N, int64_t K) {
  return swiglu_tiled(a_codes, a_scales, w_codes, w_scales, a_rows, M_total, G, N, K)
             ? grouped_tile_blocks(M_total, G, N)
             : ring_max_parts(N, G);
}

int64_t grouped_swiglu_parts_bound(int64_t M_total, int64_t N, int G) {
  const int64_t r = ring_max_parts(N, G);
  if ((M_total + G - 1) / G < GROUPED_MFMA_MIN_ROWS) return r;
  const int64_t t = grouped_tile_blocks(M_total, G, N);
  return t > r ? t : r;
}

// Most amax partials a quantize workgroup reduces by itself (8 KB of reads).
constexpr int64_t SWIGLU_INLINE_PARTS = 2048;

bool grouped_swiglu_supported(int64_t N, int64_t K, int gran, int64_t a_rows,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const uint8_t* w_codes, const uint8_t* w_scales) {
  const bool gran_ok = gran == 1 || gran == 2 || gran == 4 || gran == 8;
  return gran_ok && N % (2 * gran) == 0 && K % 256 == 0 && K >= 256 && aligned16(a_codes) &&
         aligned16(a_scales) && aligned16(w_codes) && aligned16(w_scales) &&
         a_rows * (K / 2) < ((int64_t)1 << 31) &&
         ring_lds_bytes<1, 3, 2>(K) <= RING_MAX_LDS;  // the smallest configuration fits
}

hipError_t launch_grouped_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* gsa, int64_t a_rows, const int32_t* row_index,
                                 const int32_t* offsets, int G, int64_t M_total,
                                 const uint8_t* w_codes, const uint8_t* w_scales,
                                 const float* ws2, float* h, float* gsa_h, int64_t N, int64_t K,
                                 int gran, float limit, uint32_t* partials, uint8_t* h_codes,
                                 uint8_t* h_scales, hipStream_t s) {
  GemvArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.gsa = gsa;
  a.row_index = row_index;
  a.offsets = offsets;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.ws2 = ws2;
  a.y = h;
  a.y_bf16 = 0;
  a.M = (int)M_total;
  a.N = (int)N;
  a.K = (int)K;
  a.a_rows = (int)a_rows;
  a.gran = gran;
  a.limit = limit;
  a.partials = partials;
  const int64_t mean_rows = (M_total + G - 1) / G;
  hipError_t err = hipSuccess;
  int64_t parts = 0;
  if (swiglu_tiled(a_codes, a_scales, w_codes, w_scales, a_rows, M_total, G, N, K)) {
    err = launch_grouped_gemm_swiglu(a_codes, a_scales, gsa, a_rows, row_index, offsets, G,
                                     M_total, w_codes, w_scales, ws2, h, N, K, gran, limit,
                                     partials, s);
    parts = grouped_tile_blocks(M_total, G, N);
  } else if (!launch_ring<true>(a, G, mean_rows, s, &err, &parts)) {
    return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  if (h_codes == nullptr) return launch_amax_finalize(partials, parts, gsa_h, s);
  // h's quantize as well: with few partials each quantize workgroup reduces
  // them itself (one launch), else the finalize runs first
  if (parts <= SWIGLU_INLINE_PARTS)
    return launch_quantize_finalize(h, M_total, N / 2, partials, parts, gsa_h, h_codes, h_scales,
                                    s);
  err = launch_amax_finalize(partials, parts, gsa_h, s);
  if (err != hipSuccess) return err;
  return launch_quantize(h, false, M_total, N / 2, gsa_h, h_codes, h_scales, s);
}

hipError_t launch_grouped_swiglu_l1(const uint8_t* a_codes, const uint8_t* a_scales,
                                    const float* gsa, int64_t a_rows, const int32_t* row_index,
                                    const int32_t* offsets, int G, int64_t M_total,
                                    const uint8_t* w_codes, const uint8_t* w_scales,
                                    const float* ws2, float* h, int64_t N, int64_t K, int gran,
                                    float limit, uint32_t* partials, int64_t* nparts,
                                    hipStream_t s) {
  GemvArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.gsa = gsa;
  a.row_index = row_index;
  a.offsets = offsets;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.ws2 = ws2;
  a.y = h;
  a.M = (int)M_total;
  a.N = (int)N;
  a.K = (int)K;
  a.a_rows = (int)a_rows;
  a.gran = gran;
  a.limit = limit;
  a.partials = partials;
  if (swiglu_tiled(a_codes, a_scales, w_codes, w_scales, a_rows, M_total, G, N, K)) {
    *nparts = grouped_tile_blocks(M_total, G, N);
    return launch_grouped_gemm_swiglu(a_codes, a_scales, gsa, a_rows, row_index, offsets, G,
                                      M_total, w_codes, w_scales, ws2, h, N, K, gran, limit,
                                      partials, s);
  }
  hipError_t err = hipSuccess;
  if (!launch_ring<true>(a, G, (M_total + G - 1) / G, s, &err, nparts)) return hipErrorInvalidValue;
  return err;
}

bool gemv_run_supported(int64_t M, int64_t K, const void* x, const uint8_t* w_codes,
                        const uint8_t* w_scales) {
  const int64_t nblk = M * (K / 16);
  return M >= 1 && M <= GEMV_RUN_MAX_M && K % 256 == 0 && nblk <= 2 * GEMV_MAX_WAVES * 64 &&
         M * (K / 2 + K / 16) <= GEMV_RUN_MAX_LDS && aligned16(x) && aligned16(w_codes) &&
         aligned16(w_scales);
}

template <int MP, bool XBF16, int BPT>
static hipError_t launch_run_t(const GemvArgs& a, dim3 grid, int nw, size_t lds, hipStream_t s) {
  gemv_fp4_kernel<S_GROUP, MP, true, MODE_RUN, XBF16, BPT><<<grid, nw * 64, lds, s>>>(a);
  return hipGetLastError();
}

template <int MP>
static hipError_t launch_run_mp(const GemvArgs& a, bool xbf16, int bpt, dim3 grid, int nw,
                                size_t lds, hipStream_t s) {
  if (xbf16)
    return bpt == 1 ? launch_run_t<MP, true, 1>(a, grid, nw, lds, s)
                    : launch_run_t<MP, true, 2>(a, grid, nw, lds, s);
  return bpt == 1 ? launch_run_t<MP, false, 1>(a, grid, nw, lds, s)
                  : launch_run_t<MP, false, 2>(a, grid, nw, lds, s);
}

hipError_t launch_gemv_run(const void* x, bool x_bf16, float* gsa, uint8_t* codes,
                           uint8_t* scales, const uint8_t* w_codes, const uint8_t* w_scales,
                           const float* ws2, void* y, bool y_bf16, int64_t M, int64_t N, int64_t K,
                           hipStream_t s) {
  GemvArgs a{};
  a.x = x;
  a.gsa_out = gsa;
  a.codes_out = codes;
  a.scales_out = scales;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.ws2 = ws2;
  a.y = y;
  a.y_bf16 = y_bf16 ? 1 : 0;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.a_rows = (int)M;
  const int64_t nblk = M * (K / 16);
  int nw = waves_for(K);
  while ((int64_t)nw * 64 * 2 < nblk && nw < GEMV_MAX_WAVES) ++nw;  // two blocks per thread at most
  const int bpt = nblk <= (int64_t)nw * 64 ? 1 : 2;
  const size_t lds = (size_t)(M * (K / 2 + K / 16));
  dim3 grid((unsigned)((N + 15) / 16), 1u);
  if (M <= 2) return launch_run_mp<1>(a, x_bf16, bpt, grid, nw, lds, s);
  if (M <= 4) return launch_run_mp<2>(a, x_bf16, bpt, grid, nw, lds, s);
  return launch_run_mp<8>(a, x_bf16, bpt, grid, nw, lds, s);
}

}  // namespace nvfp4
