// Fixed per-device scratch memory of the entry point that allocates nothing
// (bsa_attention_noalloc): a file-scope device array, one copy per GPU the
// library runs on, held until the process ends.  Host code must never pass
// the array's name to a kernel or a copy -- in host code it is only a
// stand-in; static_scratch() returns the device address, looked up with
// hipGetSymbolAddress once per device with that device current.
#include <mutex>

#include "bsa_internal.h"

namespace bsa {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

}  // namespace bsa
