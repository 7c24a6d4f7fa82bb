// Device scratch of the allocation-free forward (jfa_fwd_noalloc): a file-scope device
// array that replaces the caller's workspace for callers that cannot allocate device
// memory.  Each GPU holds its own copy of the array until the process ends; host code
// never passes the array's name to a kernel (in host code it is only a stand-in
// symbol) but the per-device address that hipGetSymbolAddress returns.
#include <hip/hip_runtime.h>

#include <mutex>

#include "jfa_internal.h"

namespace {

__device__ __align__(256) char scratch[jfa::kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace jfa {

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    // once per device, with that device current: its copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p % 256) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace jfa
