// Decode-shaped ternary product (M <= 64 tokens) with fused dequantization.
//
// The sum acc[m][n] = sum_k q[m][k] * t[n][k] over ternary t is the add /
// subtract / skip sum of "BitNet / Ternary / Binary - Les LLMs 1-bit" (TL;DR)
// and of the correcting reply in Hacker News Reader item 39537919: activations
// whose weight is +1 are added, those whose weight is -1 subtracted, the rest
// skipped.  Here the skip costs nothing and the add/subtract is done 1024
// weights at a time by the int8 matrix cores: each 2-bit code is moved to the
// top of its own byte, so the byte reads 64*t in {-64, 0, 64} and the matrix
// core adds or subtracts 64*q; the total is shifted right by 6 at the end
// (exact, every term is a multiple of 64).
//
// Work decomposition.  The weights are a grid of 1 KB tiles (16 rows x 256
// columns).  A wave owns NB consecutive 16-row blocks of outputs and a
// contiguous range of k-tiles; per tile it reads 16 bytes per lane (the whole
// 1 KB tile in one coalesced instruction), expands each of the four 2-bit
// fields into a 16x64 int8 operand and issues 4 * MB * NB MFMA 16x16x64 steps.
// Tile loads (and the activation operands of the same tile) are issued kU
// tiles ahead of use.  The waves of a workgroup split K and add their partial
// sums with LDS atomics; when several workgroups split K too, their sums meet
// in an int32 workspace through device-scope atomics and the last workgroup to
// arrive (a counter) dequantizes, stores y and zeroes the workspace again.
#include "bl_internal.h"

namespace bl {
namespace {

// Per token-block count MB: output blocks per wave, tiles in flight per wave
// and the largest workgroup (wider token blocks need more registers).
template <int MB> struct Shape;
template <> struct Shape<1> { static constexpr int NB = 1, U = 4, MAXW = 16; };
template <> struct Shape<2> { static constexpr int NB = 2, U = 2, MAXW = 16; };
template <> struct Shape<3> { static constexpr int NB = 2, U = 1, MAXW = 8; };
template <> struct Shape<4> { static constexpr int NB = 2, U = 1, MAXW = 8; };

inline int shape_nb(int mb) { return mb == 1 ? Shape<1>::NB : Shape<2>::NB; }
inline int shape_maxw(int mb) { return mb <= 2 ? Shape<1>::MAXW : Shape<3>::MAXW; }

struct GemvPlan {
  int MB, NB;      // 16-row token blocks, 16-row output blocks per wave
  int Nt, Kt, Ng;  // output blocks, k-tiles, output groups (Nt / NB)
  int waves, SB;   // waves per workgroup, workgroups per output group
  int tps;         // k-tiles per wave
  int64_t ws_acc_bytes, ws_bytes;
};

GemvPlan make_plan(int64_t M, int64_t N, int64_t K) {
  GemvPlan p{};
  p.MB = (int)ceil_div(M < 1 ? 1 : M, 16);
  p.NB = shape_nb(p.MB);
  p.Nt = (int)ceil_div(N, kTileN);
  p.Kt = (int)ceil_div(K, kTileK);
  p.Ng = (int)ceil_div(p.Nt, p.NB);
  // aim for about 8192 waves (32 per CU) with at least one tile each
  const int64_t units = (int64_t)p.Ng * p.Kt;
  int tpw = (int)ceil_div(units, 8192);
  if (tpw < 1) tpw = 1;
  int S = (int)ceil_div(p.Kt, tpw);
  const int maxw = shape_maxw(p.MB);
  p.waves = S < maxw ? S : maxw;
  p.SB = (int)ceil_div(S, p.waves);
  S = p.waves * p.SB;
  p.tps = (int)ceil_div(p.Kt, S);
  if (p.SB > 1) {
    p.ws_acc_bytes = (int64_t)M * p.Ng * p.NB * kTileN * 4;
    p.ws_bytes = p.ws_acc_bytes + (int64_t)p.Ng * 4;
  }
  return p;
}

template <int MB, int NB = Shape<MB>::NB, int kU = Shape<MB>::U>
__global__ __launch_bounds__(64 * Shape<MB>::MAXW) void gemv_t2_kernel(
    const int8_t* __restrict__ q, int64_t ldq, const float* __restrict__ ds, int M,
    const u4* __restrict__ packed, const float* __restrict__ beta, int N, int Nt, int Kt,
    int tps, int SB, void* __restrict__ y, int y_dtype, int32_t* __restrict__ ws_acc,
    uint32_t* __restrict__ ws_cnt) {
  constexpr int E = MB * NB * 4;  // accumulator values per lane
  __shared__ int red[E][64];

  const int lane = threadIdx.x & 63, waves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int grp = blockIdx.x / SB, sb = blockIdx.x - grp * SB;
  const int split = sb * waves + wave;
  const int k0 = split * tps;
  const int k1 = min(k0 + tps, Kt);
  const int nb0 = grp * NB;
  const int r16 = lane & 15, g4 = lane >> 4;

  v4i acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = v4i{0, 0, 0, 0};

  // Per-lane activation rows.  Lanes of token rows >= M read row M-1 instead:
  // their accumulators are never stored, so the loads need no branch.
  const int8_t* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    arow[mb] = q + (int64_t)min(mb * 16 + r16, M - 1) * ldq + 16 * g4;
  const u4* bptr[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int nb = min(nb0 + j, Nt - 1);  // blocks past Nt are masked at the store
    bptr[j] = packed + (int64_t)nb * Kt * 64 + lane;
  }

  u4 wbuf[kU][NB];
  v4i abuf[kU][MB][4];
  auto load_tile = [&](int slot, int kt) {
#pragma unroll
    for (int j = 0; j < NB; ++j) wbuf[slot][j] = __builtin_nontemporal_load(bptr[j] + (int64_t)kt * 64);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        abuf[slot][mb][i] = *reinterpret_cast<const v4i*>(arow[mb] + (int64_t)kt * kTileK + 64 * i);
  };
  auto mma_tile = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const v4i b = t2_field(wbuf[slot][j], i);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][j] = mfma16(abuf[slot][mb][i], b, acc[mb][j]);
      }
  };

  if (k0 < k1) {
    // ring of kU tiles in flight; the re-loads past the end read tile k1-1
    // again (in bounds) and are never used
#pragma unroll
    for (int u = 0; u < kU; ++u) load_tile(u, min(k0 + u, k1 - 1));
    int kt = k0;
    for (; kt + kU <= k1; kt += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        mma_tile(u);
        load_tile(u, min(kt + u + kU, k1 - 1));
      }
    }
    const int rem = k1 - kt;
#pragma unroll
    for (int u = 0; u < kU - 1; ++u)
      if (u < rem) mma_tile(u);
  }

  // ---- reduce the waves of this workgroup
  if (waves > 1) {
    for (int e = threadIdx.x; e < E * 64; e += blockDim.x) (&red[0][0])[e] = 0;
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) atomicAdd(&red[(mb * NB + j) * 4 + r][lane], acc[mb][j][r]);
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mb][j][r] = red[(mb * NB + j) * 4 + r][lane];
  }

  // ---- combine workgroups (split K across the grid)
  const int ldw = gridDim.x / SB * NB * kTileN;  // workspace row length
  if (SB > 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mb * 16 + 4 * g4 + r;
          const int n = (nb0 + j) * kTileN + r16;
          if (m < M)
            __hip_atomic_fetch_add(ws_acc + (int64_t)m * ldw + n, acc[mb][j][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    __threadfence();
    int last = 0;
    if (lane == 0)
      last = __hip_atomic_fetch_add(ws_cnt + grp, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(SB - 1);
    last = __shfl(last, 0, 64);
    if (!last) return;
    __threadfence();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mb * 16 + 4 * g4 + r;
          const int n = (nb0 + j) * kTileN + r16;
          acc[mb][j][r] = m < M ? __hip_atomic_exchange(ws_acc + (int64_t)m * ldw + n, 0, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                : 0;
        }
    if (lane == 0) __hip_atomic_store(ws_cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- dequantize and store: lane holds rows 4*g4 + r of each token block,
  //      column r16 of each output block
  const float bt = *beta;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb * 16 + 4 * g4 + r;
      if (m >= M) continue;
      const float scale = ds[m] * bt;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = (nb0 + j) * kTileN + r16;
        if (n < N) store_out(y, y_dtype, (int64_t)m * N + n, acc[mb][j][r], scale);
      }
    }
}

template <int MB>
hipError_t launch_t(const GemvPlan& p, const int8_t* q, int64_t ldq, const float* ds, int64_t M,
                    const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype,
                    void* ws, hipStream_t s) {
  int32_t* ws_acc = nullptr;
  uint32_t* ws_cnt = nullptr;
  if (p.SB > 1) {
    ws_acc = static_cast<int32_t*>(ws);
    ws_cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + p.ws_acc_bytes);
  }
  hipLaunchKernelGGL((gemv_t2_kernel<MB>), dim3((unsigned)(p.Ng * p.SB)), dim3(64 * p.waves), 0, s,
                     q, ldq, ds, (int)M, reinterpret_cast<const u4*>(packed), beta, (int)N, p.Nt,
                     p.Kt, p.tps, p.SB, y, y_dtype, ws_acc, ws_cnt);
  return hipGetLastError();
}

}  // namespace

int64_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K) { return make_plan(M, N, K).ws_bytes; }

hipError_t launch_gemv_t2(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y,
                          int y_dtype, void* ws, hipStream_t s) {
  const GemvPlan p = make_plan(M, N, K);
  switch (p.MB) {
    case 1: return launch_t<1>(p, q, ldq, ds, M, packed, beta, N, y, y_dtype, ws, s);
    case 2: return launch_t<2>(p, q, ldq, ds, M, packed, beta, N, y, y_dtype, ws, s);
    case 3: return launch_t<3>(p, q, ldq, ds, M, packed, beta, N, y, y_dtype, ws, s);
    default: return launch_t<4>(p, q, ldq, ds, M, packed, beta, N, y, y_dtype, ws, s);
  }
}

}  // namespace bl
