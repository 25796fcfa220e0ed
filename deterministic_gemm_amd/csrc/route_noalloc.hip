// route_noalloc.hip -- the library's one statically allocated device buffer,
// for dr_route_noalloc: callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc) still get the two-launch router families, whose logits kernel
// hands the logits to the selection kernel through memory.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code its
// name is only a host-side stand-in, so host code never passes it to a
// kernel: the address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept, and only that address is used.  Every
// call on a GPU shares that GPU's array and it keeps the last call's
// contents; nothing in it needs to start at zero (the logits kernel writes
// every value the selection kernel reads).  Calls that overlap on one GPU
// (two streams, two threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace drk {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // first call on this device, with it current: its copy's address
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace drk
