// Fixed device scratch for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  paged_attn_decode_noalloc keeps its split partials here
// instead of in a caller workspace.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, allocated when the code object is loaded onto that
// device and kept until the process ends.  In host code its name is only a
// host-side stand-in, never a device address, so the device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and that pointer is what kernels receive.  All calls on one device
// share the array and it keeps the last call's contents; the decode partials
// are fully written before they are read, so nothing needs clearing.  Calls
// that overlap on one device (several host threads or HIP streams at once)
// race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.hpp"

namespace pa {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];
}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -6;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -6;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace pa
