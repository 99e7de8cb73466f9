// Library-owned staging memory for rfq_linear_noalloc, the entry point for
// callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// rfq_linear stages Q(X) and Q(R) (codes and scales) in a caller-supplied
// workspace between its two kernels. The allocation-free variant stages them
// in `scratch` below instead: a file-scope device array that the code
// object's loader places on every GPU the library runs on, held until the
// process ends. In host code the name `scratch` is only a stand-in symbol,
// not a device address, so the host never passes it to a kernel or a copy:
// the first call on each device looks up that device's address once with
// hipGetSymbolAddress (the device being current) and every call uses the
// address kept for the current device.
//
// Nothing in the array has to start at zero: the quantize kernel writes
// every byte of Q(X), Q(R) and their scales that the GEMM then reads. All
// calls on one device share the array, which keeps the last call's
// contents; two calls that overlap on one GPU (on streams not ordered
// against each other) race on it.

#include <atomic>

#include "kernels.h"

namespace rfq {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(uint8_t** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<uint8_t*>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace rfq
