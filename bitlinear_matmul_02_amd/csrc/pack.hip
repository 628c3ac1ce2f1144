// Absmean ternarization and 2-bit tiled packing of latent fp32 weights
// ("Key Technologies Enabling the BitNET Family", Advanced Quantization
// Methodologies: absmean ternary weights; "BitNet / Ternary / Binary - Les
// LLMs 1-bit", Apercu de l'entrainement d'un BitLinear: beta = mean |w|,
// t = clamp(round(w / (beta + 1e-8)), -1, 1); "BitNet Technical Notes",
// Appendix: 2 bits per ternary weight).
//
// Three launches, all offline (once per weight tensor):
//   1. chunk sums: thread c adds |w| over elements [4096c, 4096c+4096) in
//      index order, in fp64;
//   2. one thread adds the chunk sums in ascending order -> beta (fp32);
//   3. one thread per packed 32-bit word ternarizes its 16 weights and writes
//      the word.  A wave writes one 256-byte quarter of a tile.
// The fixed summation order makes beta reproducible bit for bit.
//
// Binary weights (BitNet b1, "BitNet / Ternary / Binary - Les LLMs 1-bit",
// TL;DR: every weight +1 or -1) take the same beta and one bit per weight,
// 1 for w >= 0, in 16 x 512 tiles (pack_b1_kernel).
//
// Base-3 packing (pack_b3_kernel) stores the same ternary codes five to a
// byte: 16 x 320 tiles, byte i of lane L = sum_s (t + 1) * 3^s over the
// columns 64 s + 16 (L / 16) + i of row L % 16.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr float kEpsW = 1e-8f;

__global__ __launch_bounds__(256) void absmean_chunks_kernel(const float* __restrict__ w,
                                                             int64_t count, int64_t nchunks,
                                                             double* __restrict__ part) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int64_t i0 = c * kBetaChunk;
  const int64_t i1 = (i0 + kBetaChunk < count) ? i0 + kBetaChunk : count;
  double p = 0.0;
  int64_t i = i0;
  // 16-byte loads when the chunk is aligned; additions stay in index order.
  if ((reinterpret_cast<uintptr_t>(w + i0) & 15) == 0) {
    for (; i + 4 <= i1; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(w + i);
      p += fabs((double)v.x);
      p += fabs((double)v.y);
      p += fabs((double)v.z);
      p += fabs((double)v.w);
    }
  }
  for (; i < i1; ++i) p += fabs((double)w[i]);
  part[c] = p;
}

__global__ void absmean_final_kernel(const double* __restrict__ part, int64_t nchunks,
                                     int64_t count, float* __restrict__ beta) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int64_t c = 0; c < nchunks; ++c) s += part[c];
  *beta = (float)(s / (double)count);
}

__device__ inline uint32_t code2(float w, float d) {
  const float r = fminf(fmaxf(rintf(w / d), -1.0f), 1.0f);
  return (uint32_t)((int)r & 3);
}

// Word `idx` of the packed buffer: tile = idx / 256, lane L = (idx % 256) / 4,
// dword d = idx % 4.  Byte b, field i of the word is weight
// (16*nb + L%16, 256*kb + 64*i + 16*(L/16) + 4*d + b).
__global__ __launch_bounds__(256) void pack_t2_kernel(const float* __restrict__ w, int64_t N,
                                                      int64_t K, int64_t Kt,
                                                      const float* __restrict__ beta,
                                                      uint32_t* __restrict__ packed,
                                                      int64_t nwords) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nwords) return;
  const int64_t tile = idx >> 8;
  const int L = (int)((idx >> 2) & 63), d = (int)(idx & 3);
  const int64_t nb = tile / Kt, kb = tile - nb * Kt;
  const int64_t n = nb * kTileN + (L & 15);
  const int64_t kbase = kb * kTileK + 16 * (L >> 4) + 4 * d;
  const float dd = *beta + kEpsW;
  uint32_t word = 0;
  if (n < N) {
    const float* row = w + n * K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t k0 = kbase + 64 * i;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t k = k0 + b;
        if (k < K) word |= code2(row[k], dd) << (8 * b + 2 * i);
      }
    }
  }
  packed[idx] = word;
}

// Word `idx` of a B1 buffer: tile = idx / 256, lane L = (idx % 256) / 4,
// dword d = idx % 4.  Bit 16*h + j of the word is weight
// (16*nb + L%16, 512*kb + 64*(2*d + h) + 16*(L/16) + j), 1 where w >= 0.
__global__ __launch_bounds__(256) void pack_b1_kernel(const float* __restrict__ w, int64_t N, int64_t K,
                                                      int64_t Kt, uint32_t* __restrict__ packed, int64_t nwords) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nwords) return;
  const int64_t tile = idx >> 8;
  const int L = (int)((idx >> 2) & 63), d = (int)(idx & 3);
  const int64_t nb = tile / Kt, kb = tile - nb * Kt;
  const int64_t n = nb * kTileN + (L & 15);
  uint32_t word = 0;
  if (n < N) {
    const float* row = w + n * K;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t k0 = kb * 512 + 64 * (2 * d + h) + 16 * (L >> 4);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t k = k0 + j;
        if (k < K && row[k] >= 0.0f) word |= 1u << (16 * h + j);
      }
    }
  }
  packed[idx] = word;
}

// Word `idx` of a B3 buffer: tile = idx / 256, lane L = (idx % 256) / 4,
// dword d = idx % 4; byte b of the word is byte i = 4 d + b of the lane.
__global__ __launch_bounds__(256) void pack_b3_kernel(const float* __restrict__ w, int64_t N, int64_t K,
                                                      int64_t Kt, const float* __restrict__ beta,
                                                      uint32_t* __restrict__ packed, int64_t nwords) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nwords) return;
  const int64_t tile = idx >> 8;
  const int L = (int)((idx >> 2) & 63), d = (int)(idx & 3);
  const int64_t nb = tile / Kt, kb = tile - nb * Kt;
  const int64_t n = nb * kTileN + (L & 15);
  const float dd = *beta + kEpsW;
  uint32_t word = 0;
  if (n < N) {
    const float* row = w + n * K;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t v = 0, p3 = 1;
#pragma unroll
      for (int st = 0; st < 5; ++st) {
        const int64_t k = kb * kTileKB3 + 64 * st + 16 * (L >> 4) + 4 * d + b;
        if (k < K) v += (uint32_t)((int)fminf(fmaxf(rintf(row[k] / dd), -1.0f), 1.0f) + 1) * p3;
        p3 *= 3;
      }
      word |= v << (8 * b);
    }
  }
  packed[idx] = word;
}

hipError_t launch_absmean(const float* w, int64_t count, float* beta, double* partials, hipStream_t s) {
  const int64_t nchunks = ceil_div(count, kBetaChunk);
  hipLaunchKernelGGL(absmean_chunks_kernel, dim3((unsigned)ceil_div(nchunks, 256)), dim3(256), 0, s,
                     w, count, nchunks, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(absmean_final_kernel, dim3(1), dim3(64), 0, s, partials, nchunks, count, beta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_b1(const float* w, int64_t N, int64_t K, uint8_t* packed, float* beta, double* partials,
                          hipStream_t s) {
  hipError_t e = launch_absmean(w, N * K, beta, partials, s);
  if (e != hipSuccess) return e;
  const int64_t Kt = ceil_div(K, kTileKB1), Nt = ceil_div(N, kTileN);
  const int64_t nwords = Nt * Kt * (kTileBytes / 4);
  hipLaunchKernelGGL(pack_b1_kernel, dim3((unsigned)ceil_div(nwords, 256)), dim3(256), 0, s, w, N, K, Kt,
                     reinterpret_cast<uint32_t*>(packed), nwords);
  return hipGetLastError();
}

hipError_t launch_pack_b3(const float* w, int64_t N, int64_t K, uint8_t* packed, float* beta, double* partials,
                          hipStream_t s) {
  hipError_t e = launch_absmean(w, N * K, beta, partials, s);
  if (e != hipSuccess) return e;
  const int64_t Kt = ceil_div(K, kTileKB3), Nt = ceil_div(N, kTileN);
  const int64_t nwords = Nt * Kt * (kTileBytes / 4);
  hipLaunchKernelGGL(pack_b3_kernel, dim3((unsigned)ceil_div(nwords, 256)), dim3(256), 0, s, w, N, K, Kt, beta,
                     reinterpret_cast<uint32_t*>(packed), nwords);
  return hipGetLastError();
}

hipError_t launch_pack_t2(const float* w, int64_t N, int64_t K, uint8_t* packed, float* beta,
                          double* partials, hipStream_t s) {
  hipError_t e = launch_absmean(w, N * K, beta, partials, s);
  if (e != hipSuccess) return e;
  const int64_t Kt = ceil_div(K, kTileK), Nt = ceil_div(N, kTileN);
  const int64_t nwords = Nt * Kt * (kTileBytes / 4);
  hipLaunchKernelGGL(pack_t2_kernel, dim3((unsigned)ceil_div(nwords, 256)), dim3(256), 0, s, w, N, K,
                     Kt, beta, reinterpret_cast<uint32_t*>(packed), nwords);
  return hipGetLastError();
}

}  // namespace bl
