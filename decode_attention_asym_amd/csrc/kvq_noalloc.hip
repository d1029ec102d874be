// kvq_noalloc.hip -- the device scratch of kvq_decode_attn_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get their split
// partials from this file-scope array instead of a workspace argument.  Each
// device the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a stand-in for a
// device address, so its address on a device is asked for once per device
// (with that device current) and kept; only that address is ever handed to
// kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace kvq
