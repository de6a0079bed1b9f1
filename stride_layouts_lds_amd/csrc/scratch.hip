// scratch.hip -- the device scratch of sl_gemm_no_alloc: a file-scope device
// array, one copy per GPU the library runs on, held until the process ends.
// It takes the place of the caller's workspace for a split-K plan's fp32
// partial sums, so that a caller that cannot allocate device memory can
// still run those plans.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sl_kernels.hpp"

namespace sl {
namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

}  // namespace

// The device address of this GPU's scratch array.  In host code the
// array's name stands for a host-side shadow, not for device memory, so the
// address comes from the runtime, once per device with that device current,
// and is kept per device.
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace sl
