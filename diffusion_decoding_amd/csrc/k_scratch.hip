// Device scratch of the allocation-free entry point: one file-scope array,
// which the loader places in the memory of every GPU the code object is
// loaded on (each GPU holds its own copy, at its own address, until the
// process ends).  Host code must not use the array's name as a device
// address -- on the host it names a stand-in -- so the device address is
// looked up with hipGetSymbolAddress once per device (with that device
// current) and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace dg {
namespace {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return 0;
}

}  // namespace dg
