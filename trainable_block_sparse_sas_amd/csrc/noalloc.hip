// Scratch memory for the allocation-free decode call (sas_sparse_decode_noalloc):
// a fixed device array in this library's code object, one copy per GPU, held
// until the process ends.  Its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept; host code passes
// that address to kernels and never the array's name, which on the host is
// only a stand-in for the symbol.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace sas {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
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

}  // namespace sas
