// Library-owned device scratch for flashloop_attend_noalloc: callers that
// cannot allocate (code under HIP graph capture, serving loops that forbid
// allocation) pass no workspace; the attend kernels then take their partial
// results, statistics, gathered tiles and counters from this array instead.
//
// Each GPU holds its own copy of `scratch` (FLASHLOOP_STATIC_SCRATCH_BYTES)
// from the moment the library's code object loads on it until the process
// ends.  In host code the array's name is only a stand-in: its device address
// on the current GPU comes from hipGetSymbolAddress, taken once per device and
// kept.  Every call on one GPU shares the array, so calls that overlap on one
// GPU (several streams, several threads) race; the attend kernels never rely
// on its contents at entry (their counters are zeroed by the call's first
// launch), so no clearing is needed between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "flashloop.h"
#include "fl_launch.hpp"

namespace {

static __device__ __align__(256) uint8_t scratch[FLASHLOOP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace fl {

// The scratch address on the device of `st` (the current device for the null
// stream).  hipErrorInvalidValue: the stream belongs to another device than
// the current one, or the device index is beyond the table.
hipError_t static_scratch(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (st) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidValue;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace fl
