// chain_noalloc.hip -- the scratch memory of spec_verify_chain_noalloc: a file-scope device
// array that stands in for the caller's workspace, for callers that cannot allocate device
// memory. Each GPU the library runs on holds its own copy of the array until the process
// ends; every call on a GPU uses that GPU's copy, so calls that overlap on one GPU race.
#include <mutex>

#include "specv_internal.h"

// The array's name is a host-side stand-in in host code, not a device address: host code
// uses only the per-device address that chain_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[specv::kChainScratchBytes];

namespace specv {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t chain_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace specv
