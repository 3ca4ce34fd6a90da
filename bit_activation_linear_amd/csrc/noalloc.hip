// Fixed scratch for the forward entry point that allocates nothing: a
// file-scope device array of kNoAllocScratchBytes, of which each GPU the
// library runs on holds its own copy (at its own address) from the moment the
// library's code object is loaded on it until the process ends.
//
// In host code the array's name is only a host-side handle, not a device
// address. Its address on a device is looked up once per device, with that
// device current, through hipGetSymbolAddress, and only that address is ever
// handed to kernels.
#include <mutex>

#include "kernels.h"

namespace bitnet {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace bitnet
