// The library's own scratch memory for callers that cannot allocate
// (h3_dit_forward_noalloc): one static device array per GPU, part of the code
// object, so it exists on every device the library runs on until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is
// only a stand-in for the symbol): it looks up the array's device address once
// per device with hipGetSymbolAddress, with that device current, and uses that
// address everywhere.
#include <mutex>

#include "../../include/h3dit.h"
#include "launch.h"

namespace h3 {

static __device__ __align__(256) char scratch[H3_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace h3
