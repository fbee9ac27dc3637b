// cpr_static.hip -- the library-owned scratch of gdn_prefill_static: a file-scope device array that
// the code object holds on every device the library runs on, for callers that cannot allocate.
//
// In host code the array's name is only a host-side stand-in: its device address (one per device,
// the array being instantiated on each) is taken with hipGetSymbolAddress on the device's first
// use and cached, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cpr_launch.hpp"

namespace cpr {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static void* ptrs[kMaxDevices] = {};
  static std::mutex lock;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(lock);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace cpr
