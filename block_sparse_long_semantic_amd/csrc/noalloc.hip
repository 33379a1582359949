// The library's one file-scope device buffer: the workspace of infllm2_decode_step_noalloc, the
// decoding step for callers that cannot allocate device memory.  Each GPU the library runs on
// holds its own copy of `scratch` until the process ends; host code only ever passes the
// device address looked up for the current device (never the array's name, which on the host
// is a stand-in, not a device address).
#include <atomic>

#include "internal.h"

namespace infllm2 {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Zero-fill of n 32-bit words by a kernel (not a memset node, so that the step may be captured).
__global__ void __launch_bounds__(256) fill_zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

}  // namespace

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and cached; racing first calls store the same address.
hipError_t noalloc_scratch(void** ptr) {
  static std::atomic<void*> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = cached[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cached[dev].store(p, std::memory_order_relaxed);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  const int n = static_cast<int>(bytes / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_words, dim3(std::min(1024, (n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace infllm2
