// Device-resident scratch for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): bitlinear_gemv_noalloc keeps the int32 partial sums of a
// k-range split across workgroups in a fixed array that every GPU the library
// runs on holds until the process ends, instead of a caller's workspace.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is ever handed to a kernel.
//
// Contents: the product kernels take the workspace zero and leave it zero.
// The array is cleared by a fill kernel on its first use on a device and again
// after any failed launch; calls that overlap on one GPU share the array and
// race (serialize them, e.g. on one stream).
#include <atomic>
#include <mutex>

#include "bl_internal.h"

namespace bl {
namespace {

static __device__ __align__(256) uint8_t scratch[BITLINEAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;                // device address of `scratch` on this device
  std::atomic<bool> dirty{true};      // must be cleared before the next use
};
DeviceScratch g_scratch[kMaxDevices];

__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) p[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t current(DeviceScratch** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  *out = &g_scratch[dev];
  return hipSuccess;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** ptr) {
  DeviceScratch* d = nullptr;
  hipError_t e = current(&d);
  if (e != hipSuccess) return e;
  // set-up, once per device, with that device current
  std::call_once(d->once, [d] { d->err = hipGetSymbolAddress(&d->ptr, HIP_SYMBOL(scratch)); });
  if (d->err != hipSuccess) return d->err;
  if (d->dirty.exchange(false)) {
    constexpr int64_t n16 = BITLINEAR_NOALLOC_SCRATCH_BYTES / 16;
    hipLaunchKernelGGL(zero_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(d->ptr), n16);
    e = hipGetLastError();
    if (e != hipSuccess) {
      d->dirty = true;
      return e;
    }
  }
  *ptr = d->ptr;
  return hipSuccess;
}

void noalloc_mark_dirty() {
  DeviceScratch* d = nullptr;
  if (current(&d) == hipSuccess) d->dirty = true;
}

}  // namespace bl
