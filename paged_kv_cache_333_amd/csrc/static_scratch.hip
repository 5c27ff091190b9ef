// Library-owned workspace of pa_decode_split_static: a file-scope device array,
// so that call needs no allocation from its caller or from the library.
//
// Host code never passes `scratch` itself to a kernel or a copy: its name on
// the host is a stand-in, not a device address.  The device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept; every device holds its own copy of the array at its own address
// from the first lookup until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace pa {

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static std::vector<void*> addr;  // per device id
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (addr.size() <= static_cast<size_t>(dev)) addr.resize(static_cast<size_t>(dev) + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace pa
