// Device scratch of libi4s that needs no allocation: a file-scope array in
// the library's code object, for the entry point that allocates nothing
// (i4s_run_noalloc).  Its size is I4S_NOALLOC_SCRATCH_BYTES.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// array's device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to a kernel.  Each GPU holds its own copy of the array, kept
// until the process ends; every call on a GPU shares it.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "i4s_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[I4S_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

namespace i4s {

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace i4s
