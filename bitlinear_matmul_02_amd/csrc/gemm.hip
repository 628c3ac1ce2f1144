// Prefill-shaped ternary product (any number of tokens) on the int8 matrix
// cores, with fused dequantization.
//
// At many tokens the ternary product is a dense contraction, so the 2-bit
// tiles are expanded to int8 operands ({-64, 0, 64} = 64*t, see t2_field) and
// fed to MFMA 16x16x64; each matrix-core step performs the add / subtract /
// skip sum ("BitNet / Ternary / Binary - Les LLMs 1-bit", TL;DR) of 1024
// weights for 16 tokens.  The int32 total is shifted right by 6 (exact) and
// dequantized as y = acc * (ds * beta) in the epilogue.
//
// Tiling: a workgroup of 4 waves computes a 128 x 128 block of outputs; each
// wave a 64 x 64 sub-block (4 x 4 MFMA accumulators).  The k loop walks the
// 256-column weight tiles; the 16-byte tile slice of each lane is read once
// per tile and expanded in registers into four B operands (one per 2-bit
// field), the matching A operands are 16-byte loads from the int8 rows.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kBM = 128, kBN = 128;

__global__ __launch_bounds__(256) void gemm_t2_kernel(const int8_t* __restrict__ q, int64_t ldq,
                                                      const float* __restrict__ ds, int M,
                                                      const u4* __restrict__ packed,
                                                      const float* __restrict__ beta, int N,
                                                      int Nt, int Kt, void* __restrict__ y,
                                                      int y_dtype) {
  constexpr int MB = 4, NB = 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kBM + wm * 64;
  const int nb0 = (blockIdx.x * kBN + wn * 64) / kTileN;
  const int r16 = lane & 15, g4 = lane >> 4;

  v4i acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = v4i{0, 0, 0, 0};

  const int8_t* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = min(m0 + mb * 16 + r16, M - 1);  // rows past M are masked at the store
    arow[mb] = q + (int64_t)row * ldq + 16 * g4;
  }
  const u4* bptr[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) bptr[j] = packed + (int64_t)min(nb0 + j, Nt - 1) * Kt * 64 + lane;

  for (int kt = 0; kt < Kt; ++kt) {
    u4 w[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) w[j] = bptr[j][(int64_t)kt * 64];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4i a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb] = *reinterpret_cast<const v4i*>(arow[mb] + (int64_t)kt * kTileK + 64 * i);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const v4i b = t2_field(w[j], i);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][j] = mfma16(a[mb], b, acc[mb][j]);
      }
    }
  }

  const float bt = *beta;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + mb * 16 + 4 * g4 + r;
      if (m >= M) continue;
      const float scale = ds[m] * bt;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = (nb0 + j) * kTileN + r16;
        if (n < N) store_out(y, y_dtype, (int64_t)m * N + n, acc[mb][j][r], scale);
      }
    }
}

}  // namespace

int64_t gemm_ws_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_t2(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y,
                          int y_dtype, void*, hipStream_t s) {
  const int Nt = (int)ceil_div(N, kTileN), Kt = (int)ceil_div(K, kTileK);
  dim3 grid((unsigned)ceil_div(N, kBN), (unsigned)ceil_div(M, kBM));
  hipLaunchKernelGGL(gemm_t2_kernel, grid, dim3(256), 0, s, q, ldq, ds, (int)M,
                     reinterpret_cast<const u4*>(packed), beta, (int)N, Nt, Kt, y, y_dtype);
  return hipGetLastError();
}

}  // namespace bl
