// Library-owned scratch memory for the allocation-free compression entry
// point (fkv_compress_noalloc): a fixed-size device array in the code object,
// so that callers that may not allocate (code under stream capture, tight
// serving loops, harnesses that forbid hipMalloc) still get the per-layer
// workspace of the compression kernels.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a stand-in: the
// device address of a device's copy comes from hipGetSymbolAddress, called
// once per device with that device current, and only that address is ever
// handed to kernels.  Every call on one device shares that device's copy,
// so calls that overlap on one device (different streams, or threads) race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fkv_launch.h"

namespace fkv {
namespace {

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

}  // namespace

hipError_t scratch_address(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      // Device `dev` is current: this is its copy's address.
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace fkv
