// Library-owned device scratch for callers that cannot allocate.
//
// One file-scope device array; every GPU the library runs on holds its own
// copy for the life of the process.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace ssm {
namespace {

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_device_ptr(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace ssm
