// A library-held verification workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops and harnesses that
// forbid allocation).  It backs specdec_verify_greedy_noalloc.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "specdec.h"

namespace sd {

// The array lives in the code object: every device the library runs on holds
// its own copy, at its own address, until the process ends.  In host code this
// name is only a handle for the symbol lookup below, never an address.
static __device__ __align__(256) unsigned char scratch[SPECDEC_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` on device d, once looked up
}  // namespace

// Device address of the current device's copy of `scratch`.  The first call on
// a device (with that device current) takes the address with
// hipGetSymbolAddress and clears the array with a fill kernel on `s`: the
// loader zero-fills it too, and greedy verification leaves every word it uses
// zeroed again, so it stays cleared between calls.
hipError_t static_scratch(void **out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    e = launch_zero(p, SPECDEC_STATIC_SCRATCH_BYTES, s);
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace sd
