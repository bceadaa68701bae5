// fa_noalloc.hip - the fp32 dQ workspace of atomic mode as a static device
// array, for the entry point that allocates nothing (fa_bwd_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code
// its name is only a host-side stand-in, so the device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept; kernels receive that address, never the name.  Every call on one GPU
// shares that GPU's array and leaves the last call's contents in it.

#include <mutex>

#include "fa_kernels.h"
#include "../../include/fa.h"

namespace fa {
namespace {

static_assert(FA_STATIC_WORKSPACE_BYTES % 256 == 0, "whole 256-byte units");
static __device__ __align__(256) float scratch[FA_STATIC_WORKSPACE_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
float* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, once known

// zero n floats (n a multiple of 4) with 16-byte stores
__global__ void __launch_bounds__(256) zero_kernel(float* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x)
    ((f32x4*)p)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace

hipError_t static_workspace(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = (float*)ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_zero(float* p, size_t bytes, hipStream_t s) {
  const int64_t n4 = (int64_t)(bytes / 16);
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n4);
  return hipGetLastError();
}

}  // namespace fa
