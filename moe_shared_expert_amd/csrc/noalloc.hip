// Scratch memory of the allocation-free forward entry point: one statically sized
// device array per GPU, in place of a caller-provided workspace.
//
// Host code must never pass the array's name to a kernel or a copy: in host code it is
// a host-side stand-in, not a device address.  Its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and cached; every later
// use goes through that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "smlp.h"

namespace {

__device__ __attribute__((aligned(256))) char scratch[SMLP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace smlp {

int noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return (int)hipSuccess;
}

}  // namespace smlp
