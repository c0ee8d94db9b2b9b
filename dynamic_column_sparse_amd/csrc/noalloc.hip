// Library-owned scratch for the allocation-free entry point
// (chipmunk_sparse_mlp_delta_noalloc): a file-scope device array that every
// GPU the library runs on holds from module load until the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device
// address.  Its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and cached; kernels are
// handed that address, as they are handed a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace chipmunk {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace chipmunk
