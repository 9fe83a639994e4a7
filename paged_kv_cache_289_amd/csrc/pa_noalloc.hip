// Device scratch of paged_attn_decode_noalloc: a file-scope array that every
// GPU the library runs on holds until the process ends, so that the call
// allocates nothing.  The array's name is a host-side stand-in, not a device
// address: the address of each device's copy is looked up once per device,
// with that device current, and only that address is handed to kernels.
#include <mutex>

#include "pa_internal.h"

namespace {

__device__ __align__(256) char scratch[pa::kScratchBytes];

std::mutex g_mu;
void* g_ptr[pa::kMaxDevices] = {};

}  // namespace

namespace pa {

hipError_t scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace pa
