// router.hip -- the dense router's expert choice on the gate linear's
// logits: sqrt(softplus(logit)) + per-expert bias, then the top k experts
// (archived_plans/CORRECTNESS_BACKLOG.md, section 5 "Router", and the
// commit message on the router gate in single_shot_inference.py of commit
// 107d62d: the logit already carries gsa * gsb from the linear's epilogue).
//
// One workgroup per row.  Its 256 threads form the activations and the
// selection keys (order-preserving bits of the value) in LDS -- the
// activation is most of the arithmetic, so it is spread over four waves.
// Then one wave holds the keys of experts l, l + 64, ... in lane l, and
// each of the k rounds finds the largest live key (DPP within rows of 16
// lanes, the scalar unit across rows), takes the lowest expert index that
// holds it from ballots, and retires that expert.  No LDS traffic inside
// the rounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace nvfp4 {

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

template <int NV>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ src, int nsrc, const float* __restrict__ gsa_p,
    const float* __restrict__ ws2_p, float* __restrict__ logits, const float* __restrict__ bias,
    int M, int N, int k, int32_t* __restrict__ idx, float* __restrict__ score) {
#pragma clang fp contract(off)
  __shared__ float s_lds[64 * NV];
  __shared__ uint32_t key_lds[64 * NV];
  const int m = blockIdx.x;
  const int64_t MN = (int64_t)M * N;
  // the activation of expert j by thread j % 256 (all its loads first)
  constexpr int PT = (64 * NV + 255) / 256;
  float zv[PT], bv[PT];
#pragma unroll
  for (int t = 0; t < PT; ++t) {
    const int j = min((int)threadIdx.x + 256 * t, N - 1);
    const int64_t e = (int64_t)m * N + j;
    if (nsrc == 0) {
      zv[t] = src[e];
    } else {  // split-K partials: their sum in split order, then the scale
      float p[GEMM_MAX_SPLITS];
#pragma unroll
      for (int z = 0; z < GEMM_MAX_SPLITS; ++z) p[z] = z < nsrc ? src[z * MN + e] : 0.0f;
      float v = p[0];
#pragma unroll
      for (int z = 1; z < GEMM_MAX_SPLITS; ++z)
        if (z < nsrc) v += p[z];
      zv[t] = v * (gsa_p[0] * ws2_p[0]);
      if ((int)threadIdx.x + 256 * t < N) logits[e] = zv[t];
    }
    bv[t] = bias ? bias[j] : 0.0f;
  }
#pragma unroll
  for (int t = 0; t < PT; ++t) {
    const int j = threadIdx.x + 256 * t;
    if (j < 64 * NV) {
      const float sj = sqrt_softplus(zv[t]);
      s_lds[j] = sj;
      key_lds[j] = j < N ? order_key(sj + bv[t]) : 0u;
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  uint32_t key[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t) key[t] = key_lds[lane + 64 * t];
  int mine = 0;  // lane r keeps the expert of round r
  for (int r = 0; r < k; ++r) {
    // the largest live key: each lane's own, then the max within rows of 16
    // lanes (DPP: swap neighbours, swap pairs, mirror halves, mirror the
    // row), then across the four rows on the scalar unit
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
    // first t with a hit and the lowest lane in that t's ballot.  k <= N, so
    // a live key (nonzero) is left in every round.
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
    idx[(int64_t)m * k + lane] = mine;
    score[(int64_t)m * k + lane] = s_lds[mine];
  }
}

hipError_t launch_router_topk(const float* src, int nsrc, const float* gsa, const float* ws2,
                              float* logits, const float* bias, int64_t M, int64_t N, int k,
                              int32_t* idx, float* score, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (nsrc < 0 || nsrc > GEMM_MAX_SPLITS) return hipErrorInvalidValue;
  const dim3 grid((unsigned)M);
  const int nv = (int)((N + 63) / 64);
#define ROUTER_LAUNCH(V)                                                                       \
  router_topk_kernel<V><<<grid, 256, 0, s>>>(src, nsrc, gsa, ws2, logits, bias, (int)M, (int)N, \
                                             k, idx, score)
  if (nv <= 1)
    ROUTER_LAUNCH(1);
  else if (nv <= 2)
    ROUTER_LAUNCH(2);
  else if (nv <= 4)
    ROUTER_LAUNCH(4);
  else if (nv <= 8)
    ROUTER_LAUNCH(8);
  else if (nv <= 16)
    ROUTER_LAUNCH(16);
  else
    return hipErrorInvalidValue;
#undef ROUTER_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
