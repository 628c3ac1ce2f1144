// Elementwise glue between the BitLinears of a decoder layer.
//
// Feed-forward activation ("Key Technologies Enabling the BitNET Family",
// Architectural Innovations and Optimizations: squared ReLU in the
// feed-forward layers): h = ReLU(g)^2 * u, with r = g if g > 0 else +0, then
// (r * r) * u, two fp32 roundings in that order.  Streams 12 bytes per
// element; 16-byte vectors when all three pointers allow it.
#include <algorithm>

#include "bl_internal.h"

namespace bl {
namespace {

__device__ inline float relu2_mul1(float g, float u) {
  const float r = g > 0.0f ? g : 0.0f;
  return __fmul_rn(__fmul_rn(r, r), u);
}

template <bool VEC>
__global__ __launch_bounds__(256) void relu2_mul_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                        float* h, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if constexpr (VEC) {
    const int64_t n4 = count >> 2;
    for (int64_t j = i; j < n4; j += stride) {
      const float4 a = reinterpret_cast<const float4*>(g)[j];
      const float4 b = reinterpret_cast<const float4*>(u)[j];
      reinterpret_cast<float4*>(h)[j] =
          make_float4(relu2_mul1(a.x, b.x), relu2_mul1(a.y, b.y), relu2_mul1(a.z, b.z), relu2_mul1(a.w, b.w));
    }
    i += n4 << 2;  // the last count % 4 elements
    if (i < count) h[i] = relu2_mul1(g[i], u[i]);
  } else {
    for (; i < count; i += stride) h[i] = relu2_mul1(g[i], u[i]);
  }
}

}  // namespace

hipError_t launch_relu2_mul(const float* g, const float* u, int64_t count, float* h, hipStream_t s) {
  const bool vec = ((reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(u) |
                     reinterpret_cast<uintptr_t>(h)) & 15) == 0;
  const int64_t items = vec ? ceil_div(count, 4) : count;
  const unsigned blocks = (unsigned)std::min<int64_t>(std::max<int64_t>(ceil_div(items, 256), 1), 2048);
  if (vec)
    hipLaunchKernelGGL((relu2_mul_kernel<true>), dim3(blocks), dim3(256), 0, s, g, u, h, count);
  else
    hipLaunchKernelGGL((relu2_mul_kernel<false>), dim3(blocks), dim3(256), 0, s, g, u, h, count);
  return hipGetLastError();
}

}  // namespace bl
