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
#include "router.hpp"

namespace nvfp4 {

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
  router_rounds<NV>(key_lds, s_lds, k, idx + (int64_t)m * k, score + (int64_t)m * k);
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
