// The workspace of mcs_select_noalloc: a fixed array inside the library, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy (MCS_NOALLOC_SCRATCH_BYTES) until the process ends.
// In host code its name is only a stand-in for the device object: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and only that address is handed to the kernels.  Calls on
// one device share the array, so calls that overlap on one GPU race; every
// region the selection reads is written earlier in the same call, so nothing
// needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "mcs.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MCS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up once per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t mcs::noalloc_scratch(void** out) { return scratch_address(out); }
