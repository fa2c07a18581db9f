// The fixed device scratch of the allocation-free forward entry point
// (poetx_linear_fwd_noalloc), for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy for the life of the process. In host code the array's name is
// only a host-side stand-in, so its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and that address
// is what the entry point passes to the kernels as their workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "poetx.h"

namespace poetx {
namespace {

__device__ __align__(256) unsigned char scratch[POETX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace poetx
