// Fixed scratch memory of the allocation-free GEMM entry point (w12_gemm_noalloc in w12.h).
//
// The array below is device memory that every GPU the library runs on holds once its code object
// is loaded, until the process ends.  In host code its name is only a host-side stand-in, never a
// device address: the address is looked up with hipGetSymbolAddress, once per device with that
// device current, and only that pointer is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "w12_launch.hpp"

namespace w12 {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t fixed_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

}  // namespace w12
