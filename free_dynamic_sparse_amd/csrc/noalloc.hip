// Scratch memory of the allocation-free forward (solattn_fwd_noalloc): the
// fused kernel's work-queue counters in a file-scope device array instead of
// a caller's workspace, for callers that cannot allocate device memory.
//
// Every GPU the library runs on holds its own copy of the array until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address, so the device address is looked up once per device (with
// that device current) and only that address is ever handed to a kernel.
// Every call on one GPU shares its array; the launch clears the counters
// in-stream before the fused kernel runs, so calls that overlap on one GPU
// race.

#include <mutex>

#include "launch.hpp"
#include "noalloc.hpp"

namespace solattn {

// 8 work-queue counters, one 128-byte line apart: the fused forward's whole
// workspace (fwd_workspace_bytes()).
static __device__ __align__(256) uint32_t scratch[256];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device, once looked up
}  // namespace

size_t noalloc_scratch_bytes() { return sizeof(scratch); }

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
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

}  // namespace solattn
