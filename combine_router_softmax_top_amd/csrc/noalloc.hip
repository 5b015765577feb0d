// The dispatch's scratch memory for callers that cannot allocate: one
// file-scope device array per GPU, held until the process ends.
//
// moe_dispatch's kernels keep a per-chunk expert histogram, the rank of every
// assignment inside its chunk and per-chunk row bases in a caller-owned
// workspace.  moe_dispatch_noalloc runs the same kernels on this array
// instead.  Nothing in it has to start at zero (every entry the kernels read
// was written earlier in the same call), and calls that overlap on one GPU
// share it, so they race.
#include <mutex>

#include "moe_internal.h"

namespace moe {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each GPU

}  // namespace

// The array's address on the current device.  In host code `scratch` names a
// host-side stand-in, never a device address, so kernels are only ever given
// what hipGetSymbolAddress returns (each device holds its own copy).
hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
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

}  // namespace moe
