// Scratch memory for the entry points that allocate nothing: a fixed array in
// this library's device code, one copy per GPU, alive until the process ends.
//
// In host code the array's name is only a stand-in for the device symbol, not
// a device address; its address on the current device is looked up once per
// device with hipGetSymbolAddress and that pointer is what the kernels get.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current (hipGetDevice above)
  std::call_once(g_once[dev], [dev] {
    g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}
