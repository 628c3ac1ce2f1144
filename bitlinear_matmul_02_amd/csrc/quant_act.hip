// Per-token absmax int8 activation quantization
// ("Key Technologies Enabling the BitNET Family", Advanced Quantization
// Methodologies: 8-bit activations by absmax, per token).
//
// One workgroup of 256 threads per token row.  Pass 1 finds gamma = max|x|
// with a wavefront butterfly (DPP/ds_swizzle via __shfl_xor) and one LDS
// exchange between the four waves; pass 2 re-reads the row (an L2 hit) and
// writes q = clamp(rint(x * (127/g)), -127, 127), g = max(gamma, 1e-5), eight
// elements per thread per step, plus zero padding up to the row stride.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr float kEpsX = 1e-5f;

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int XDT>
__device__ inline float load_x(const void* x, int64_t i) {
  if constexpr (XDT == BITLINEAR_BF16)
    return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
  else
    return static_cast<const float*>(x)[i];
}

// Eight consecutive elements starting at i (caller guarantees 16-byte
// alignment for bf16 / 16-byte alignment of each half for fp32).
template <int XDT>
__device__ inline void load_x8(const void* x, int64_t i, float (&v)[8]) {
  if constexpr (XDT == BITLINEAR_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ inline int quant1(float x, float qs) {
  const float r = rintf(x * qs);
  return (int)fminf(fmaxf(r, -127.0f), 127.0f);
}

template <int XDT, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const void* __restrict__ x,
                                                              int64_t K, int64_t ldq,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ ds,
                                                              int32_t* __restrict__ rowsum) {
  __shared__ float red_f[kThreads / 64];
  __shared__ int red_i[kThreads / 64];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = m * K;

  // pass 1: gamma = max |x|
  float amax = 0.0f;
  if constexpr (VEC) {
    for (int64_t k = 8 * (int64_t)tid; k < K; k += 8 * kThreads) {
      float v[8];
      load_x8<XDT>(x, base + k, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
  } else {
    for (int64_t k = tid; k < K; k += kThreads) amax = fmaxf(amax, fabsf(load_x<XDT>(x, base + k)));
  }
  amax = wave_max(amax);
  if (lane == 0) red_f[wave] = amax;
  __syncthreads();
  float gamma = red_f[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) gamma = fmaxf(gamma, red_f[w]);

  const float g = fmaxf(gamma, kEpsX);
  const float qs = 127.0f / g;  // IEEE division (correctly rounded build)

  // pass 2: quantize, 8 elements -> one 8-byte store
  int8_t* qrow = q + m * ldq;
  int sum = 0;
  for (int64_t k = 8 * (int64_t)tid; k < ldq; k += 8 * kThreads) {
    int c[8];
    if (VEC && k + 8 <= K) {
      float v[8];
      load_x8<XDT>(x, base + k, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = quant1(v[j], qs);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = (k + j < K) ? quant1(load_x<XDT>(x, base + k + j), qs) : 0;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= (uint32_t)(c[j] & 0xff) << (8 * j);
      hi |= (uint32_t)(c[4 + j] & 0xff) << (8 * j);
      sum += c[j] + c[4 + j];
    }
    *reinterpret_cast<uint2*>(qrow + k) = make_uint2(lo, hi);
  }
  if (rowsum != nullptr) {
    sum = wave_sum(sum);
    if (lane == 0) red_i[wave] = sum;
  }
  __syncthreads();
  if (tid == 0) {
    ds[m] = g / 127.0f;
    if (rowsum != nullptr) {
      int s = 0;
      for (int w = 0; w < kThreads / 64; ++w) s += red_i[w];
      rowsum[m] = s;
    }
  }
}

}  // namespace

hipError_t launch_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldq,
                            int8_t* q, float* ds, int32_t* rowsum, hipStream_t s) {
  const bool vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  dim3 grid((unsigned)M), block(kThreads);
  if (x_dtype == BITLINEAR_BF16) {
    if (vec)
      hipLaunchKernelGGL((quant_act_kernel<BITLINEAR_BF16, true>), grid, block, 0, s, x, K, ldq, q, ds, rowsum);
    else
      hipLaunchKernelGGL((quant_act_kernel<BITLINEAR_BF16, false>), grid, block, 0, s, x, K, ldq, q, ds, rowsum);
  } else {
    if (vec)
      hipLaunchKernelGGL((quant_act_kernel<BITLINEAR_F32, true>), grid, block, 0, s, x, K, ldq, q, ds, rowsum);
    else
      hipLaunchKernelGGL((quant_act_kernel<BITLINEAR_F32, false>), grid, block, 0, s, x, K, ldq, q, ds, rowsum);
  }
  return hipGetLastError();
}

}  // namespace bl
