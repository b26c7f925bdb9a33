// The static device scratch of pa_unified_attention_noalloc: split partials,
// per-row part counts and the longest-first unit order of a call live in one
// file-scope device array instead of hipMalloc'd memory, for callers that
// cannot allocate (code under stream capture, tight serving loops).
//
// Every GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// kept.  Calls on one GPU share the array, so calls that overlap on one GPU
// race; nothing in it needs to start at zero (every slot a kernel reads was
// written earlier in the same call).

#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

__device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace pa
