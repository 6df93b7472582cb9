// Library-owned decode scratch for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): a file-scope device array that every GPU the library
// runs on holds from module load until the process ends.
//
// In host code the array's name is only a host-side stand-in for the symbol;
// its device address is taken once per device, with that device current,
// through hipGetSymbolAddress, and only that address is ever handed to
// kernels.  Every call on one GPU shares that GPU's array, which keeps the
// contents of the last call; calls that overlap on one GPU (several streams
// or threads) race on it.
#include <mutex>

#include "pa_internal.h"

namespace pa {

constexpr size_t kNoallocScratchBytes = size_t(32) << 20;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pa
