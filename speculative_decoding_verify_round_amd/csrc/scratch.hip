// The library's own device scratch, for the entry point that allocates nothing
// (spec_verify_head_noalloc): a file-scope device array per GPU, looked up once per
// device and kept until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace sv {

constexpr int kMaxDevices = 64;

// In host code this name is a stand-in for the device array, not its address: kernels and
// copies get the address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

int static_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -1;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  *bytes = kStaticScratchBytes;
  return 0;
}

}  // namespace sv
