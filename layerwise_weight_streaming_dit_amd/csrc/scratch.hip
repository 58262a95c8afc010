// Library-owned device scratch for callers that cannot allocate device memory
// at call time (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc): the per-forward activation workspace of
// dlo_forward_static lives in this file-scope array instead of the caller's
// arena.  Each GPU the library runs on holds its own copy, at its own
// address, from the first use on that device until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory; the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current and cached here.
#include <mutex>

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace dlo {

namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[device] = p;
  }
  *out = g_ptr[device];
  return hipSuccess;
}

}  // namespace dlo
