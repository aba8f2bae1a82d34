// Device scratch of the allocation-free fused layer (moe_fused_fp8_noalloc).
//
// Callers that cannot allocate device memory -- code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc -- get the
// layer's workspace (routing arrays, the fp8 intermediate and its scales,
// the weighted expert outputs) from this file-scope array instead.  Each GPU
// the library runs on holds its own copy, at its own address, until the
// process ends.  In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device, with that device
// current, and that address is what the launches receive.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fp8moe.h"
#include "launch.h"

namespace fp8moe {

static __device__ __align__(256) uint8_t scratch[FP8MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex lock;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> g(lock);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // device `dev` is current
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace fp8moe
