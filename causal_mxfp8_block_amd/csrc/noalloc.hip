// noalloc.hip -- the static device workspace of mxfa_attn_fwd_noalloc: the forward's K and V
// encodings in a file-scope device array instead of caller-provided memory, for callers that cannot
// allocate (code under graph capture, tight serving loops). Every device the library runs on holds
// one copy of the array until the process ends; concurrent calls on one device share it and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace mxfa {

__device__ __align__(256) uint8_t scratch[kNoallocWorkspaceBytes];

// The array's device address on the current device. The host-side name `scratch` is only a stand-in
// for the symbol, never a device address: the address is looked up once per device, with that device
// current, and kept.
hipError_t noalloc_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace mxfa
