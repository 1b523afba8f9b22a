// Library-owned scratch memory for mla_decode_paged_noalloc: a fixed device array per GPU, so
// that a decode can run where the caller cannot allocate (inside HIP graph capture, in a tight
// serving loop, under a harness that forbids allocation).
//
// `scratch` is a file-scope __device__ array: every device the library runs on holds its own
// copy, resident until the process ends.  In host code its name is only a host-side stand-in,
// so the device address is taken once per device with hipGetSymbolAddress (with that device
// current) and cached; launches receive that address, never the symbol itself.  Calls that
// share one GPU share its array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_internal.hpp"

namespace mla {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];   // device address of `scratch` per device, null = not set up
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
