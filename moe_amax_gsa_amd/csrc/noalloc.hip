// noalloc.hip -- nvfp4_linear_run_noalloc: nvfp4_linear_run for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Its scratch -- the amax partials
// of the two-phase amax and the split-K partial sums of the tiled linear --
// lives in one file-scope device array of NVFP4_NOALLOC_SCRATCH_BYTES,
// which each GPU the library runs on holds until the process ends.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on a device comes from hipGetSymbolAddress, taken
// once per device (with that device current) on the first call there, and
// only that address is passed to kernels.  Every call on a GPU shares that
// GPU's array; calls that overlap on one GPU (two streams, or two threads)
// race on it.  Nothing in it has to start at zero: each kernel writes every
// partial it later reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/nvfp4.h"
#include "launch.hpp"

#define NVFP4_API extern "C" __attribute__((visibility("default")))

namespace {

static __device__ __align__(256) uint8_t scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
void* scratch_ptr[MAX_DEVICES];  // per device, set once under scratch_mu
std::mutex scratch_mu;

// The current device's address of `scratch` (looked up on its first use).
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

NVFP4_API int nvfp4_linear_run_noalloc(const void* x, int x_dtype, float* gsa, uint8_t* codes,
                                       uint8_t* scales, const uint8_t* w_codes,
                                       const uint8_t* w_scales, const float* ws2, void* y,
                                       int y_dtype, int64_t M, int64_t N, int64_t K,
                                       void* stream) {
  const int st = nvfp4::linear_run_check(x, x_dtype, gsa, codes, scales, w_codes, w_scales, ws2,
                                         y, y_dtype, M, N, K);
  if (st != NVFP4_OK || M == 0) return st;
  if (nvfp4_workspace_bytes(NVFP4_OP_LINEAR_RUN, M, N, K, 1) > NVFP4_NOALLOC_SCRATCH_BYTES)
    return NVFP4_ERR_SCRATCH;
  void* ptr = nullptr;
  if (scratch_on_current_device(&ptr) != hipSuccess) return NVFP4_ERR_LAUNCH;
  return nvfp4_linear_run(x, x_dtype, gsa, codes, scales, w_codes, w_scales, ws2, y, y_dtype, M,
                          N, K, ptr, NVFP4_NOALLOC_SCRATCH_BYTES, stream);
}
