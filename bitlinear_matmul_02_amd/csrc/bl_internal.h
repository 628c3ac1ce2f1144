// Internal declarations shared by the HIP translation units of libbitlinear.
// gfx950 only: wave64, int8 MFMA 16x16x64, correctly rounded fp32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "bitlinear.h"

namespace bl {

// Geometry of the 2-bit tiled weight format: a tile is 16 rows x 256 columns,
// 1024 bytes, read by one wave as 64 lanes x 16 bytes.
constexpr int kTileN = 16;
constexpr int kTileK = 256;
constexpr int kTileBytes = 1024;
constexpr int kBetaChunk = 4096;
// LDS a decode workgroup may use for its int8 activation rows (each row is
// act_stride(K) + 16 bytes); with its 4 KB reduction buffer it stays < 64 KB.
constexpr int kTileKB1 = 512;  // columns of a 1 KB binary (B1) tile
constexpr int kTileKB3 = 320;  // columns of a 1 KB base-3 (B3) tile
constexpr int kActAlign = 512;  // int8 activation rows are padded to a multiple of this
constexpr int64_t kDecodeLdsBytes = BITLINEAR_DECODE_MAX_ACT_BYTES;
constexpr int kXDtypeMask = BITLINEAR_X_RMSNORM - 1;  // x_dtype without its flags
constexpr int kGemvMaxSeg = BITLINEAR_MULTI_MAX;       // BitLinears per multi launch

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- launches
// Each returns hipSuccess or the launch error; arguments are already valid.
hipError_t launch_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldq,
                            int8_t* q, float* ds, int32_t* rowsum, hipStream_t s);

hipError_t launch_pack_t2(const float* w, int64_t N, int64_t K, uint8_t* packed, float* beta,
                          double* partials, hipStream_t s);

// Decode-shaped product (M <= 64).  `ws` may be null when gemv_ws_bytes is 0.
int64_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_t2(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y,
                          int y_dtype, void* ws, hipStream_t s);

// Host model of the decode kernel's global read extents (fmt 0 ternary 2-bit,
// 1 binary, 2 base-3; int8 rows of ldq bytes).
void gemv_read_extent(int64_t M, int64_t N, int64_t K, int fmt, int64_t ldq, int64_t* act_end, int64_t* w_end);

// The device array behind bitlinear_gemv_noalloc (zero on return, or an
// error): its address on the current device, cleared first when needed.
hipError_t noalloc_scratch(hipStream_t s, void** ptr);
// After a failed launch that used the array: clear it before its next use.
void noalloc_mark_dirty();

// Decode product of 1-4 BitLinears sharing int8 inputs (or a gated pair)
// whose last workgroup requantizes output 0 (or h) for the next BitLinear:
// as launch_gemv_multi followed by launch_quant_act of y[0] (fp32 rows).
// `ws` holds a zeroed 4-byte arrival counter, left zero.
hipError_t launch_decode_rq(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K, int count,
                            const uint8_t* const* packed, const float* const* beta, const int64_t* N, void* const* y,
                            int y_dtype, bool glu, int8_t* next_q, int64_t next_ldq, float* next_ds, bool next_norm,
                            void* ws, hipStream_t s);

// Fused decode: per-token quantization of x inside the product kernel.
bool decode_fused_fits(int64_t M, int64_t K);
hipError_t launch_decode_t2(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* packed,
                            const float* beta, int64_t N, void* y, int y_dtype, hipStream_t s);

// Prefill-shaped product (any M).
int64_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_t2(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y,
                          int y_dtype, void* ws, hipStream_t s);

hipError_t launch_gemv_multi(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K, int count,
                             const uint8_t* const* packed, const float* const* beta, const int64_t* N, void* const* y,
                             int y_dtype, bool glu, hipStream_t s);
hipError_t launch_decode_multi(const void* x, int x_dtype, int64_t M, int64_t K, int count,
                               const uint8_t* const* packed, const float* const* beta, const int64_t* N,
                               void* const* y, int y_dtype, bool glu, hipStream_t s);

hipError_t launch_pack_b1(const float* w, int64_t N, int64_t K, uint8_t* packed, float* beta, double* partials,
                          hipStream_t s);
hipError_t launch_gemv_b1(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M,
                          int64_t K, const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype,
                          hipStream_t s);

hipError_t launch_gemm_b1(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype, hipStream_t s);

hipError_t launch_pack_b3(const float* w, int64_t N, int64_t K, uint8_t* packed, float* beta, double* partials,
                          hipStream_t s);
hipError_t launch_gemv_b3(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M,
                          int64_t K, const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype,
                          hipStream_t s);

hipError_t launch_train_forward(const uint16_t* x, int64_t M, int64_t K, const uint8_t* packed, const float* beta,
                                int64_t N, float* y, hipStream_t s);
hipError_t launch_train_dx(const uint16_t* dy, int64_t M, int64_t N, const uint8_t* packed, const float* beta,
                           int64_t K, float* dx, hipStream_t s);
hipError_t launch_train_dw(const uint16_t* dy, const uint16_t* x, int64_t M, int64_t N, int64_t K, float* dw,
                           hipStream_t s);

hipError_t launch_relu2_mul(const float* g, const float* u, int64_t count, float* h, hipStream_t s);

// ------------------------------------------------------- device helpers
// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Field i of four packed words as MFMA int8 operand bytes: each output byte is
// 64 * t (t in {-1, 0, 1}) because the 2-bit two's-complement code is moved to
// the top two bits of its byte and the rest is masked off.
__device__ inline v4i t2_field(const u4 w, int i) {
  const int sh = 6 - 2 * i;
  v4i r;
  r.x = (int)((w.x << sh) & 0xC0C0C0C0u);
  r.y = (int)((w.y << sh) & 0xC0C0C0C0u);
  r.z = (int)((w.z << sh) & 0xC0C0C0C0u);
  r.w = (int)((w.w << sh) & 0xC0C0C0C0u);
  return r;
}

// One 16x16x64 int8 matrix-core step: acc += A(16x64) * B(64x16).
__device__ inline v4i mfma16(v4i a, v4i b, v4i acc) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
}

// One 32x32x32 int8 matrix-core step: acc += A(32x32) * B(32x32).  Lane l
// holds row l % 32 of A / column l % 32 of B, bytes j of k = 16 * (l / 32) + j;
// output element e of lane l is D[8 * (e / 4) + 4 * (l / 32) + e % 4][l % 32].
__device__ inline v16i mfma32(v4i a, v4i b, v16i acc) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc, 0, 0, 0);
}

// Integer maximum / sum over the 64 lanes of a wave, returned to every lane;
// all 64 lanes must be active.  Both operations are order-free, so the
// result equals any other reduction order: DPP swaps within quads
// (quad_perm 1,0,3,2 and 2,3,0,1), rotations by 4 and 8 within each row of
// 16 lanes, then the four row results through readlane.  This replaces a
// chain of six LDS-crossbar shuffles by four DPP moves.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}
// fp64 sum over the 64 lanes of a wave by the same DPP pattern (each double
// moved as two dwords), returned to every lane.  Unlike the integer forms the
// result depends on the association order; the order is fixed: within each
// row of 16 lanes, lane 0's ((quad sums 0 + 3) + (2 + 1)) after the quad
// swaps, then rows 0 + 1 + 2 + 3 in that order.
template <int CTRL>
__device__ inline double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ inline double readlane_f64(double v, int lane) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ inline double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x124>(v);
  v += dpp_f64<0x128>(v);
  return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}
__device__ inline int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// LDS race self-test.  A build compiled with -DBL_LDS_POISON (the library's
// own build never defines it) fills the LDS of every kernel that stages data
// there with a poison pattern before the first use, and the prefill GEMM
// poisons each staging buffer again once it has been consumed.  A read of LDS
// that no thread of the workgroup wrote in this launch and stage (a missing
// barrier, a wrong offset) then returns the pattern instead of a previous
// launch's or stage's bytes, which can be the right ones when the same call
// repeats, and the result no longer matches.
#ifdef BL_LDS_POISON
constexpr bool kLdsPoison = true;
#else
constexpr bool kLdsPoison = false;
#endif
constexpr uint32_t kLdsPoisonWord = 0xA5A5A5A5u;  // int8 -91; fp32 about -2.9e-16

// Poison `bytes` (a multiple of 4) of LDS at p, strided over the workgroup's
// threads; the caller adds the barrier.
__device__ inline void lds_poison(void* p, int bytes) {
  uint32_t* w = static_cast<uint32_t*>(p);
  for (int i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = kLdsPoisonWord;
}

// Raises a kernel's dynamic LDS limit on the current device, once per device
// (the attribute belongs to the device that is current when it is set).
struct LdsLimit {
  std::atomic<uint64_t> done{0};  // bit d: raised on device d
  std::mutex mu;
};
inline hipError_t ensure_lds_limit(LdsLimit& l, const void* func, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  const uint64_t bit = uint64_t(1) << dev;
  if (l.done.load(std::memory_order_acquire) & bit) return hipSuccess;
  std::lock_guard<std::mutex> g(l.mu);
  if (l.done.load(std::memory_order_relaxed) & bit) return hipSuccess;
  e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) l.done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Tile index of workgroup b when T tiles are dealt round-robin to the 8 XCDs
// (XCD x receives blocks x, x + 8, ...): XCD x gets the contiguous tiles
// [start(x), start(x) + count(x)), so its L2 sees neighbouring tiles.
__device__ inline int xcd_tile(int b, int T) {
  const int x = b & 7, i = b >> 3;
  int start = 0;
  for (int j = 0; j < x; ++j) start += (T - j + 7) >> 3;
  return start + i;
}

// Dequantize one accumulator (scaled by 64 by t2_field) and store it.
__device__ inline void store_out(void* y, int y_dtype, int64_t idx, int acc64, float scale) {
  const int acc = acc64 >> 6;  // exact: every term is a multiple of 64
  if (y_dtype == BITLINEAR_I32) {
    static_cast<int32_t*>(y)[idx] = acc;
  } else {
    const float v = (float)acc * scale;
    if (y_dtype == BITLINEAR_F32)
      static_cast<float*>(y)[idx] = v;
    else if (y_dtype == BITLINEAR_F32_ADD)
      static_cast<float*>(y)[idx] = __fadd_rn(static_cast<const float*>(y)[idx], v);
    else
      static_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
  }
}

// store_out with the output type fixed at compile time (epilogues that
// dispatch on the type once, outside their loops).
template <int YD>
__device__ inline void store_out_t(void* y, int64_t idx, int acc64, float scale) {
  const int acc = acc64 >> 6;  // exact: every term is a multiple of 64
  if constexpr (YD == BITLINEAR_I32) {
    static_cast<int32_t*>(y)[idx] = acc;
  } else {
    const float v = (float)acc * scale;
    if constexpr (YD == BITLINEAR_F32)
      static_cast<float*>(y)[idx] = v;
    else if constexpr (YD == BITLINEAR_F32_ADD)
      static_cast<float*>(y)[idx] = __fadd_rn(static_cast<const float*>(y)[idx], v);
    else
      static_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------- row requantization
// Per-token absmax quantization of one fp32 row of K values by one wave, with
// the standalone quantizer's arithmetic ("Key Technologies Enabling the BitNET
// Family", Advanced Quantization Methodologies): gamma = max |x| on the
// sign-cleared bit patterns (exact in any order); with `norm` the row is
// RMS-normalized first (S = sum x^2 in fp64, each square exact, summed per
// lane in index order then across the wave by a fixed butterfly;
// r = 1 / sqrt((float)(S / K) + 1e-5); the quantizer sees fl(x * r), whose
// maximum is fl(gamma * r)); g = max(gamma, 1e-5), q = rint(fl(x * (127 / g)))
// by the 1.5 * 2^23 magic add (|x * qs| <= 127 (1 + 2^-23), so no clamp acts),
// padding columns [K, ldq) written 0, ds = g / 127.  Rows whose length is a
// multiple of 4 and 16-byte aligned are read as 16-byte pieces (two passes:
// statistics, then codes), others element by element.
__device__ inline uint32_t rq_qbyte(float x, float qs) {
  return __float_as_uint(__fadd_rn(__fmul_rn(x, qs), 12582912.0f)) & 0xffu;
}

__device__ inline void wave_quant_row_f32(const float* x, int K, bool norm, int8_t* q, int64_t ldq, float* ds) {
  const int lane = threadIdx.x & 63;
  const bool vec = (K % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  const int n4 = vec ? K / 4 : 0;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  uint32_t amax = 0;
  double s2 = 0.0;
#pragma unroll 8
  for (int i = lane; i < n4; i += 64) {
    const float4 v = x4[i];
    amax = max(max(amax, __float_as_uint(v.x) & 0x7fffffffu), __float_as_uint(v.y) & 0x7fffffffu);
    amax = max(max(amax, __float_as_uint(v.z) & 0x7fffffffu), __float_as_uint(v.w) & 0x7fffffffu);
    if (norm) {
      s2 += (double)v.x * (double)v.x;
      s2 += (double)v.y * (double)v.y;
      s2 += (double)v.z * (double)v.z;
      s2 += (double)v.w * (double)v.w;
    }
  }
  for (int k = 4 * n4 + lane; k < K; k += 64) {  // element path (rows that are not 16-byte pieces)
    const float v = x[k];
    amax = max(amax, __float_as_uint(v) & 0x7fffffffu);
    if (norm) s2 += (double)v * (double)v;
  }
  amax = wave_max_u32(amax);
  float gamma = __uint_as_float(amax), rn = 1.0f;
  if (norm) {
    s2 = wave_sum_f64(s2);
    rn = 1.0f / sqrtf((float)(s2 / (double)K) + 1e-5f);
    gamma = __fmul_rn(gamma, rn);
  }
  const float g = fmaxf(gamma, 1e-5f);
  const float qs = 127.0f / g;  // IEEE division
  auto code = [&](float v) { return rq_qbyte(norm ? __fmul_rn(v, rn) : v, qs); };
#pragma unroll 8
  for (int i = lane; i < n4; i += 64) {
    const float4 v = x4[i];
    *reinterpret_cast<uint32_t*>(q + 4 * (int64_t)i) = code(v.x) | (code(v.y) << 8) | (code(v.z) << 16) | (code(v.w) << 24);
  }
  for (int64_t k = 4 * (int64_t)n4 + 4 * lane; k < ldq; k += 256) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (k + j < K) w |= code(x[k + j]) << (8 * j);
    *reinterpret_cast<uint32_t*>(q + k) = w;
  }
  if (lane == 0) *ds = g / 127.0f;
}

}  // namespace bl
