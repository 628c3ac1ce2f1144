// Per-token absmax int8 activation quantization
// ("Key Technologies Enabling the BitNET Family", Advanced Quantization
// Methodologies: 8-bit activations by absmax, per token).
//
// One workgroup per token row.  Each thread loads its 16-byte pieces of the
// row (8 bf16 or 4 fp32 values) once and keeps up to kHold of them in
// registers: the row maximum of |x| is taken on the sign-cleared bit patterns
// (packed 16-bit integer max for bf16), reduced across the wave with DPP
// moves and across waves through LDS; then every held piece is
// quantized, q = rint(x * (127 / g)), g = max(gamma, 1e-5), and stored as
// int8 (zero padding up to the row stride).  Rows that are not whole 16-byte
// pieces (unaligned x, or K not a multiple of the piece) take an element
// path.  Long rows get 1024 threads, short ones 256.
//
// Optionally the row is RMS-normalized first (gain 1; "Key Technologies
// Enabling the BitNET Family", Architectural Innovations and Optimizations:
// RMSNorm is the normalization): S = sum x^2 in fp64 (squares exact),
// r = 1 / sqrt((float)(S / K) + 1e-5) in fp32, and the quantizer sees
// fl(x * r).  Its maximum is fl(gamma * r) exactly, because rounding is
// monotone, so gamma is still taken on the raw row.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr float kEpsX = 1e-5f;
constexpr float kEpsNorm = 1e-5f;
constexpr int kHold = 4;  // pieces per thread kept in registers

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t piece_absmax_bits(const u4 v, bool bf16) {
  if (bf16) {
    us2 m = __builtin_bit_cast(us2, v[0] & 0x7fff7fffu);
    m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, v[1] & 0x7fff7fffu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, v[2] & 0x7fff7fffu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, v[3] & 0x7fff7fffu));
    return (uint32_t)(m.x > m.y ? m.x : m.y) << 16;
  }
  return max(max(v[0] & 0x7fffffffu, v[1] & 0x7fffffffu), max(v[2] & 0x7fffffffu, v[3] & 0x7fffffffu));
}

// q = rint(x * qs) as a byte.  |x * qs| <= 127 * (1 + 2^-23) since |x| <= g
// and qs = fl(127 / g): adding 1.5 * 2^23 rounds the product to the nearest
// integer, ties to even, into the low mantissa bits, and the clamp to
// [-127, 127] never acts.  Separate multiply and add roundings.
__device__ inline uint32_t qbyte(float x, float qs) {
  return __float_as_uint(__fadd_rn(__fmul_rn(x, qs), 12582912.0f)) & 0xffu;
}

// Quantize one piece; returns the codes' sum and writes 8 (bf16) or 4 bytes.
__device__ inline int piece_quant_store(const u4 v, bool bf16, float qs, int8_t* dst) {
  int sum = 0;
  if (bf16) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t b0 = qbyte(__uint_as_float(v[2 * h] << 16), qs);
      const uint32_t b1 = qbyte(__uint_as_float(v[2 * h] & 0xffff0000u), qs);
      const uint32_t b2 = qbyte(__uint_as_float(v[2 * h + 1] << 16), qs);
      const uint32_t b3 = qbyte(__uint_as_float(v[2 * h + 1] & 0xffff0000u), qs);
      w[h] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      sum += (int)(int8_t)b0 + (int)(int8_t)b1 + (int)(int8_t)b2 + (int)(int8_t)b3;
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
    const uint32_t b0 = qbyte(__uint_as_float(v[0]), qs), b1 = qbyte(__uint_as_float(v[1]), qs);
    const uint32_t b2 = qbyte(__uint_as_float(v[2]), qs), b3 = qbyte(__uint_as_float(v[3]), qs);
    *reinterpret_cast<uint32_t*>(dst) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    sum = (int)(int8_t)b0 + (int)(int8_t)b1 + (int)(int8_t)b2 + (int)(int8_t)b3;
  }
  return sum;
}

__device__ inline float load_x(const void* x, bool bf16, int64_t i) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[i]) : static_cast<const float*>(x)[i];
}

// Sum of squares of one piece's values, in fp64 (each square is exact).
__device__ inline double piece_sumsq(const u4 v, bool bf16) {
  double s = 0.0;
  if (bf16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = __uint_as_float(v[j] << 16), hi = __uint_as_float(v[j] & 0xffff0000u);
      s += lo * lo;
      s += hi * hi;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = __uint_as_float(v[j]);
      s += a * a;
    }
  }
  return s;
}

// r = 1 / sqrt(mean square + eps), fp32 (correctly rounded division and root).
__device__ inline float rms_scale(double sumsq, int64_t K) {
  const float ms = (float)(sumsq / (double)K);
  return 1.0f / sqrtf(ms + kEpsNorm);
}

// Apply the normalization to a piece (fp32 multiply per value); the result
// is an fp32 piece (bf16 input widens to two fp32 pieces: lo, hi).
__device__ inline u4 scale_f32_piece(const u4 v, float r) {
  return u4{__float_as_uint(__fmul_rn(__uint_as_float(v[0]), r)), __float_as_uint(__fmul_rn(__uint_as_float(v[1]), r)),
            __float_as_uint(__fmul_rn(__uint_as_float(v[2]), r)), __float_as_uint(__fmul_rn(__uint_as_float(v[3]), r))};
}

// Block-wide max of non-negative float bit patterns / sum of ints via LDS.
template <int NT>
__device__ inline uint32_t block_max(uint32_t v, uint32_t* slots) {
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = slots[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = max(r, slots[w]);
  return r;
}

template <int NT>
__device__ inline int block_sum(int v, int* slots) {
  v = wave_sum_i32(v);
  if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r += slots[w];
  return r;
}

template <int NT>
__device__ inline double block_sum_f64(double v, double* slots) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r += slots[w];
  return r;
}

// Quantize one piece after normalization: bf16 values widen exactly to fp32
// and are scaled there; writes 8 (bf16) or 4 bytes.
__device__ inline int piece_quant_store_norm(const u4 v, bool bf16, float r, float qs, int8_t* dst) {
  if (bf16) {
    const u4 lo = scale_f32_piece(u4{v[0] << 16, v[0] & 0xffff0000u, v[1] << 16, v[1] & 0xffff0000u}, r);
    const u4 hi = scale_f32_piece(u4{v[2] << 16, v[2] & 0xffff0000u, v[3] << 16, v[3] & 0xffff0000u}, r);
    return piece_quant_store(lo, false, qs, dst) + piece_quant_store(hi, false, qs, dst + 4);
  }
  return piece_quant_store(scale_f32_piece(v, r), false, qs, dst);
}

template <int NT, bool VEC, bool NORM>
__global__ __launch_bounds__(NT) void quant_act_kernel(const void* __restrict__ x, int bf16i, int64_t K,
                                                       int64_t ldq, int8_t* __restrict__ q,
                                                       float* __restrict__ ds, int32_t* __restrict__ rowsum) {
  __shared__ uint32_t slots_max[NT / 64];
  __shared__ int slots_sum[NT / 64];
  __shared__ double slots_sq[NORM ? NT / 64 : 1];
  if constexpr (kLdsPoison) {  // LDS self-test builds
    lds_poison(slots_max, (int)sizeof(slots_max));
    lds_poison(slots_sum, (int)sizeof(slots_sum));
    lds_poison(slots_sq, (int)sizeof(slots_sq));
    __syncthreads();
  }
  const bool bf16 = bf16i != 0;
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  int8_t* qrow = q + m * ldq;
  float g;
  int sum = 0;
  if constexpr (VEC) {
    const int per16 = bf16 ? 8 : 4;
    const int np = (int)(K / per16);  // pieces in the row
    const u4* src = reinterpret_cast<const u4*>(static_cast<const char*>(x) + m * K * (bf16 ? 2 : 4));
    u4 v[kHold];
#pragma unroll
    for (int r = 0; r < kHold; ++r) v[r] = src[min(tid + r * NT, np - 1)];  // duplicates never stored
    uint32_t amax = 0;
    double sq = 0.0;
#pragma unroll
    for (int r = 0; r < kHold; ++r) {
      amax = max(amax, piece_absmax_bits(v[r], bf16));
      if (NORM && tid + r * NT < np) sq += piece_sumsq(v[r], bf16);  // duplicates excluded
    }
    for (int c = tid + kHold * NT; c < np; c += NT) {
      amax = max(amax, piece_absmax_bits(src[c], bf16));
      if (NORM) sq += piece_sumsq(src[c], bf16);
    }
    float gamma = __uint_as_float(block_max<NT>(amax, slots_max));
    float rn = 1.0f;
    if constexpr (NORM) {
      rn = rms_scale(block_sum_f64<NT>(sq, slots_sq), K);
      gamma = __fmul_rn(gamma, rn);  // = max |fl(x * r)|
    }
    g = fmaxf(gamma, kEpsX);
    const float qs = 127.0f / g;  // IEEE division
    auto quant = [&](const u4 p, int c) {
      int8_t* dst = qrow + (int64_t)c * per16;
      return NORM ? piece_quant_store_norm(p, bf16, rn, qs, dst) : piece_quant_store(p, bf16, qs, dst);
    };
#pragma unroll
    for (int r = 0; r < kHold; ++r) {
      const int c = tid + r * NT;
      if (c < np) sum += quant(v[r], c);
    }
    for (int c = tid + kHold * NT; c < np; c += NT) sum += quant(src[c], c);
    for (int64_t k = K + 4 * (int64_t)tid; k < ldq; k += 4 * NT) *reinterpret_cast<uint32_t*>(qrow + k) = 0u;
  } else {
    float amax = 0.0f;
    double sq = 0.0;
    for (int64_t k = tid; k < K; k += NT) {
      const float xv = load_x(x, bf16, m * K + k);
      amax = fmaxf(amax, fabsf(xv));
      if (NORM) sq += (double)xv * (double)xv;
    }
    float gamma = __uint_as_float(block_max<NT>(__float_as_uint(amax), slots_max));
    float rn = 1.0f;
    if constexpr (NORM) {
      rn = rms_scale(block_sum_f64<NT>(sq, slots_sq), K);
      gamma = __fmul_rn(gamma, rn);
    }
    g = fmaxf(gamma, kEpsX);
    const float qs = 127.0f / g;
    for (int64_t k = 4 * (int64_t)tid; k < ldq; k += 4 * NT) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k + j < K) {
          const float xv = load_x(x, bf16, m * K + k + j);
          const uint32_t b = qbyte(NORM ? __fmul_rn(xv, rn) : xv, qs);
          w |= b << (8 * j);
          sum += (int)(int8_t)b;
        }
      *reinterpret_cast<uint32_t*>(qrow + k) = w;
    }
  }
  if (rowsum != nullptr) sum = block_sum<NT>(sum, slots_sum);
  if (tid == 0) {
    ds[m] = g / 127.0f;
    if (rowsum != nullptr) rowsum[m] = sum;
  }
}

template <int NT, bool NORM>
void launch_nt(const void* x, int bf16, int64_t M, int64_t K, int64_t ldq, int8_t* q, float* ds, int32_t* rowsum,
               bool vec, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((quant_act_kernel<NT, true, NORM>), dim3((unsigned)M), dim3(NT), 0, s, x, bf16, K, ldq, q, ds,
                       rowsum);
  else
    hipLaunchKernelGGL((quant_act_kernel<NT, false, NORM>), dim3((unsigned)M), dim3(NT), 0, s, x, bf16, K, ldq, q, ds,
                       rowsum);
}

template <bool NORM>
void launch_norm(const void* x, int bf16, int64_t M, int64_t K, int64_t ldq, int8_t* q, float* ds, int32_t* rowsum,
                 bool vec, hipStream_t s) {
  const int per16 = bf16 ? 8 : 4;
  // 1024 threads once the row has more pieces than 256 threads hold
  if (K / per16 > 256 * kHold)
    launch_nt<1024, NORM>(x, bf16, M, K, ldq, q, ds, rowsum, vec, s);
  else
    launch_nt<256, NORM>(x, bf16, M, K, ldq, q, ds, rowsum, vec, s);
}

}  // namespace

hipError_t launch_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldq,
                            int8_t* q, float* ds, int32_t* rowsum, hipStream_t s) {
  const bool bf16 = (x_dtype & kXDtypeMask) == BITLINEAR_BF16;
  const bool norm = (x_dtype & BITLINEAR_X_RMSNORM) != 0;
  const int per16 = bf16 ? 8 : 4;
  const bool vec = (K % per16 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  if (norm)
    launch_norm<true>(x, bf16, M, K, ldq, q, ds, rowsum, vec, s);
  else
    launch_norm<false>(x, bf16, M, K, ldq, q, ds, rowsum, vec, s);
  return hipGetLastError();
}

}  // namespace bl
