// Device scratch of the allocation-free backward entry point
// (dash_attn_bwd_qk_noalloc in api.cpp).
//
// One file-scope device array per GPU, of kNoallocScratchBytes, holds the
// whole workspace of a backward call (fp32 dQ accumulator, Delta,
// semaphores, error word, scratch tiles), the call's step lists, and a word
// that records a semaphore give-up.  It is allocated when this file's code
// object is loaded (the first use of the entry point in the process) and
// stays until the process ends.  Host code never uses the array's name as an
// address: its device address is fetched once per device with
// hipGetSymbolAddress, with that device current, and that pointer is what the
// kernels, copies and fills receive.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "kernels.hpp"

namespace dash {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::map<int, char*> g_scratch_ptr;  // device -> address of that device's `scratch`

}  // namespace

hipError_t noalloc_scratch(int dev, char** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev) return hipErrorInvalidDevice;  // the caller makes `dev` current
    char* p = nullptr;
    e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256) return hipErrorInvalidSymbol;
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace dash
