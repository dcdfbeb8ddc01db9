// probe.hip -- measurement probes used by the benchmark only (they are not
// part of the layer's C ABI in include/nvfp4.h).  They bound a kernel's time
// by measurement:
//   probe_empty   an empty kernel with a given grid: in a graph of
//                 back-to-back launches, the per-launch floor of that grid;
//   probe_stream  a read-only pass over two byte ranges with a given grid,
//                 each workgroup reading its contiguous slice of both with
//                 16-byte nontemporal loads: the time a weight-streaming
//                 kernel of that grid needs just to bring its bytes in.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

__global__ void probe_empty_kernel() {}

__device__ __forceinline__ uint32_t xor_slice(const uint4* __restrict__ p, int64_t n16,
                                              int64_t per_wg) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int64_t b = (int64_t)blockIdx.x * per_wg;
  const int64_t e = b + per_wg < n16 ? b + per_wg : n16;
  uint32_t acc = 0;
  // eight loads a thread in flight before any is used
  for (int64_t i0 = b + threadIdx.x; i0 < e; i0 += 8 * (int64_t)blockDim.x) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + u * (int64_t)blockDim.x;
      v[u] = __builtin_nontemporal_load((const u32x4*)(p + (i < e ? i : b)));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * (int64_t)blockDim.x < e) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  return acc;
}

// out holds one word per wave of the grid: the xor of what the wave read
// (kept so that the loads are not removed).
__global__ void probe_stream_kernel(const uint4* __restrict__ a, int64_t a16, int64_t a_per,
                                    const uint4* __restrict__ b, int64_t b16, int64_t b_per,
                                    uint32_t* __restrict__ out) {
  uint32_t acc = xor_slice(a, a16, a_per) ^ xor_slice(b, b16, b_per);
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0)
    out[(int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

PROBE_API int probe_empty(int grid, int threads, void* stream) {
  if (grid < 1 || threads < 1 || threads > 1024) return -2;
  probe_empty_kernel<<<grid, threads, 0, (hipStream_t)stream>>>();
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// a and b 16-byte aligned, a_bytes and b_bytes multiples of 16; out holds
// grid * (threads / 64) words; threads a multiple of 64.
PROBE_API int probe_stream(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes,
                           int grid, int threads, uint32_t* out, void* stream) {
  if (grid < 1 || threads < 64 || threads > 1024 || threads % 64 != 0) return -2;
  if (a_bytes < 0 || b_bytes < 0 || a_bytes % 16 != 0 || b_bytes % 16 != 0) return -2;
  if (((uintptr_t)a | (uintptr_t)b) & 15u) return -5;
  if (out == nullptr || (a_bytes > 0 && a == nullptr) || (b_bytes > 0 && b == nullptr)) return -1;
  const int64_t a16 = a_bytes / 16, b16 = b_bytes / 16;
  const int64_t a_per = (a16 + grid - 1) / grid, b_per = (b16 + grid - 1) / grid;
  probe_stream_kernel<<<grid, threads, 0, (hipStream_t)stream>>>(
      (const uint4*)a, a16, a_per, (const uint4*)b, b16, b_per, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
