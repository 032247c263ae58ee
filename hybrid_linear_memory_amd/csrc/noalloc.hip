// Scratch memory of the entry point that allocates nothing (arl2_read_noalloc):
// a file-scope device array, of which each GPU the library runs on holds its
// own copy until the process ends. Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the device symbol): the
// device address of the current device's copy is looked up once per device
// with hipGetSymbolAddress and kept, and callers use that address.
#include <mutex>

#include "arl2_internal.h"

namespace arl2 {
namespace {
constexpr size_t kNoallocScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
}  // namespace
}  // namespace arl2

static __device__ __align__(256) char scratch[arl2::kNoallocScratchBytes];

namespace arl2 {

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));     // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace arl2
