// router.hpp -- the dense router's expert choice, shared by the standalone
// choice kernel and the gate linear's last workgroup (one launch for few
// rows): sqrt(softplus(logit)) + per-expert bias, then the top k experts
// (archived_plans/CORRECTNESS_BACKLOG.md, section 5 "Router"; the logit
// already carries gsa * gsb from the linear's epilogue, as the router gate's
// commit message in single_shot_inference.py of commit 107d62d states).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int ROUTER_LDS_EXPERTS = 1024;

// softplus(z) = max(z, 0) + log1p(exp(-|z|)): log(1 + exp(z)) without
// overflow for large z and without losing the tail for very negative z.
__device__ __forceinline__ float sqrt_softplus(float z) {
  const float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
  return sqrtf(sp);
}

// Order-preserving map of a finite float to a nonzero u32 (key 0 marks a
// retired or absent expert); -0 and +0 map to one key.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One wave (lane = 0..63) picks the k experts of largest key among the
// N <= 64 NV keys in key_lds (expert j = lane + 64 t in lane `lane`), best
// first, the lower expert index first among equal keys: idx_out[r] and
// score_out[r] = s_lds[expert] for r < k.  Each round: every lane's best live
// key, a DPP max within rows of 16 lanes, the four rows' maxima on the
// scalar unit, and ballots for the lowest index holding it.
template <int NV>
__device__ __forceinline__ void router_rounds(const uint32_t* key_lds, const float* s_lds, int k,
                                              int32_t* idx_out, float* score_out) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t) key[t] = key_lds[lane + 64 * t];
  int mine = 0;  // lane r keeps the expert of round r
  for (int r = 0; r < k; ++r) {
    uint32_t x = 0u;
#pragma unroll
    for (int t = 0; t < NV; ++t) x = max(x, key[t]);
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));
    const uint32_t w = max(max((uint32_t)__builtin_amdgcn_readlane((int)x, 0),
                               (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
                           max((uint32_t)__builtin_amdgcn_readlane((int)x, 32),
                               (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
    // the lowest expert index holding it: expert j = lane + 64 t, so the
    // first t with a hit and the lowest lane in that t's ballot; k <= N, so
    // a live (nonzero) key is left in every round
    int jw = 0;
#pragma unroll
    for (int t = NV - 1; t >= 0; --t) {
      const uint64_t b = __ballot(key[t] == w);
      if (b) jw = 64 * t + __builtin_ctzll(b);
    }
#pragma unroll
    for (int t = 0; t < NV; ++t)
      if (64 * t + lane == jw) key[t] = 0u;
    if (lane == r) mine = jw;
  }
  if (lane < k) {
    idx_out[lane] = mine;
    score_out[lane] = s_lds[mine];
  }
}

// The choice for rows 0..M-1 of logits (M, N) by the whole workgroup
// (blockDim.x threads, a multiple of 64): scores and keys into LDS by all
// threads, then wave 0 runs the rounds.  N <= 1024, 1 <= k <= min(N, 64).
// COHERENT: the logits are read with device-coherent loads (other
// workgroups of this launch wrote them).
template <bool COHERENT>
__device__ __forceinline__ void router_choose_rows(const float* logits, int M, int N, int k,
                                                   const float* bias, int32_t* idx,
                                                   float* score) {
#pragma clang fp contract(off)
  __shared__ float s_lds[ROUTER_LDS_EXPERTS];
  __shared__ uint32_t key_lds[ROUTER_LDS_EXPERTS];
  // the rounds read 64 keys per slice for a power-of-two number of slices:
  // every one of them is written (absent experts get key 0)
  const int nv0 = (N + 63) / 64;
  const int nv = nv0 <= 1 ? 1 : nv0 <= 2 ? 2 : nv0 <= 4 ? 4 : nv0 <= 8 ? 8 : 16;
  for (int m = 0; m < M; ++m) {
    for (int j = threadIdx.x; j < 64 * nv; j += blockDim.x) {
      const float* zp = logits + (int64_t)m * N + min(j, N - 1);
      const float z = COHERENT ? __hip_atomic_load(zp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : *zp;
      const float sj = sqrt_softplus(z);
      s_lds[j] = sj;
      key_lds[j] = j < N ? order_key(sj + (bias ? bias[j] : 0.0f)) : 0u;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      int32_t* io = idx + (int64_t)m * k;
      float* so = score + (int64_t)m * k;
      if (nv <= 1)
        router_rounds<1>(key_lds, s_lds, k, io, so);
      else if (nv <= 2)
        router_rounds<2>(key_lds, s_lds, k, io, so);
      else if (nv <= 4)
        router_rounds<4>(key_lds, s_lds, k, io, so);
      else if (nv <= 8)
        router_rounds<8>(key_lds, s_lds, k, io, so);
      else
        router_rounds<16>(key_lds, s_lds, k, io, so);
    }
    __syncthreads();
  }
}

}  // namespace nvfp4
