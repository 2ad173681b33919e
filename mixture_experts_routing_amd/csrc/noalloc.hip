// Static device scratch for moe_forward_noalloc: the workspace of a whole moe_forward call
// (routing outputs, intermediate, accumulator) in a file-scope device array, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Each device the library runs on holds its own copy of
// the array from module load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address
// comes from hipGetSymbolAddress, taken once per device with that device current, and only
// that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
