// Fixed device scratch for the entry point that allocates nothing
// (kvc_window_scores_noalloc): callers that cannot allocate device memory, such
// as code under stream capture or a serving loop that forbids allocation.
//
// The scratch is one file-scope device array.  Host code never uses the array's
// name as a device address: the address of each device's copy is looked up once
// per device with hipGetSymbolAddress (that device current) and kept here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kvc_launch.h"

namespace kvc {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      // the device is current (hipGetDevice above): this is its copy's address
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace kvc
