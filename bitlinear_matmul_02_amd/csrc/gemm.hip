// Prefill-shaped ternary product (any number of tokens) on the int8 matrix
// cores, with fused dequantization.
//
// At many tokens the ternary product is a dense contraction, so the 2-bit
// tiles are expanded to int8 operands ({-64, 0, 64} = 64*t, see t2_field) and
// fed to MFMA 32x32x32; each matrix-core step performs the add / subtract /
// skip sum ("BitNet / Ternary / Binary - Les LLMs 1-bit", TL;DR) of 1024
// weights for 32 tokens.  The int32 total is shifted right by 6 (exact) and
// dequantized as y = acc * (ds * beta) in the epilogue.
//
// Why 32x32x32: on gfx950 one wave per SIMD issuing 32x32x32 int8 steps
// sustains ~4.1 POPS, the 16x16x64 form only ~1.6-2.7 POPS at that occupancy.
//
// Operands from the 2-bit tile format (16 rows x 256 columns per 1 KB tile,
// lane L = 16*g4 + r of a tile holds row r, columns 64*i + 16*g4 + 0..15 of
// field i): for the 32x32x32 step s (columns 32*s .. 32*s + 31 of the tile),
// lane (n = l % 32, g = l / 32) needs row n of the two 16-row tiles at
// columns 32*s + 16*g + 0..15, which is field s/2 of tile lane
// 16*(2*(s%2) + g) + n%16.  So each lane reads two 16-byte chunks per
// 256-column step (chunk h = s % 2) and expands field f for steps 2f and 2f+1.
//
// Tiling.  A workgroup of 8 waves (2 x 4) computes a BM x BN block of outputs
// (tokens x weight rows), each wave (BM/2) x (BN/4); two waves per SIMD let
// one wave's loads, LDS traffic and operand expansion overlap the other's
// matrix-core work.  Per 256-column k-step the workgroup needs the BM x 256
// int8 activation slab and the BN/16 weight tiles (BN x 64 bytes):
//   * both are requested D k-steps ahead into a register ring (activation
//     slab first: vmcnt retires in order) and written, one k-step ahead of
//     use and interleaved with the MFMAs, into the free half of
//     double-buffered LDS slabs; weight tiles are loaded once per workgroup
//     and shared by the waves in LDS;
//   * 16-byte piece c of activation row r sits in slot r*16 + (c ^ (r & 15)),
//     so the 32 rows a matrix-core operand reads fall on different banks;
//     weight tiles keep their 1 KB lane-major layout (conflict-free reads);
//   * each MFMA step's next operands (LDS reads, 2-bit expansion) are issued
//     while the current step's MFMAs run.
// Binary weights (BitNet b1, "BitNet / Ternary / Binary - Les LLMs 1-bit",
// TL;DR: weights +1 or -1) use 16 x 512 tiles of one bit per weight (format
// B1): a 256-column k-step reads dwords 2 (kt % 2) and 2 (kt % 2) + 1 of
// every lane of the tile, i.e. an 8-byte half of each lane's chunk.  Step s
// of the k-step takes, from tile lane 16 * (2 (s % 2) + g) + n % 16, the 16
// bits of dword s / 4, half (s / 2) % 2; they become 16 bytes in {0, 1} and
// the epilogue takes 2 * sum(q * b) - rowsum(q).
//
// Workgroups are numbered so that each of the 8 XCDs (blocks are dealt to
// them round-robin) works on a contiguous run of output tiles, walked in
// groups of 4 token blocks along N, which share both operands in its L2.
//
// Up to 64 tokens (decode with a batch) the blocks are 64 x 128, and when
// that leaves fewer workgroups than compute units the k-steps are split
// across S workgroups per block: each writes its int32 sums to a workspace
// slice [S][M][N] and a second kernel adds the S slices and dequantizes.
// Up to 32 tokens on wide outputs, 32 x 128 blocks split each k-step's
// matrix-core steps between two halves of the workgroup instead (four waves
// each, one 32 x 32 tile per wave), which add their sums in LDS: no
// workspace and no second launch.  Integer sums are exact in any order, so
// every split gives the unsplit result.
#include <type_traits>

#include "bl_internal.h"

namespace bl {
namespace {

template <int BM, int BN, int FMT = 0, int KS = 1>
struct GemmTile {
  static constexpr int WGK = KS;                       // waves along k (halves of each k-step's MFMA steps)
  static constexpr int WGM = BM >= 64 ? 2 : 1;         // waves along M
  static constexpr int WGN = 8 / (WGM * WGK);          // waves along N
  static constexpr int NT = 64 * WGM * WGN * WGK;     // threads per workgroup
  static constexpr int SPW = 8 / WGK;                 // MFMA steps per wave per k-step
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // per-wave block
  static constexpr int MB = WM / 32, NB = WN / 32;    // 32x32 MFMA tiles per wave
  static constexpr int SLAB_A = BM * kTileK;          // activation slab bytes
  static constexpr int TB = FMT ? kTileBytes / 2 : kTileBytes;  // weight bytes per 16-row tile per k-step
  static constexpr int SLAB_B = BN / kTileN * TB;     // weight slab bytes
  static constexpr int BP = FMT ? 8 : 16;             // bytes per weight piece
  static constexpr int PA = SLAB_A / 16 / NT;         // 16-byte pieces per thread
  static constexpr int PB = SLAB_B / BP / NT;
  static constexpr int LDS = 2 * (SLAB_A + SLAB_B);   // double-buffered
};

// Step s of a B1 chunk pair: 16 bits -> 16 bytes in {0, 1} (bit j -> byte j).
__device__ inline v4i b1_bytes(uint32_t bits16) {
  v4i r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = (int)((((bits16 >> (4 * q)) & 0xFu) * 0x00204081u) & 0x01010101u);
  return r;
}

template <int BM, int BN, int D, int FMT, bool SPLIT, int KS = 1>
__global__ __launch_bounds__(512) void gemm_t2_kernel(const int8_t* __restrict__ q, int64_t ldq,
                                                      const float* __restrict__ ds,
                                                      const int32_t* __restrict__ rowsum, int M,
                                                      const uint8_t* __restrict__ packed,
                                                      const float* __restrict__ beta, int N, int Nt,
                                                      int Kt, int KtW, int tiles_n, void* __restrict__ y,
                                                      int y_dtype, int splits, int32_t* __restrict__ part) {
  using G = GemmTile<BM, BN, FMT, KS>;
  static_assert(KS == 1 || !SPLIT, "one split of k at a time");
  using BT = typename std::conditional<FMT != 0, uint2, u4>::type;  // one weight piece
  constexpr int MB = G::MB, NB = G::NB;
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  // LDS: activation halves [0, 2 SLAB_A), then weight halves
  auto slabA = [&](int buf) { return lds + buf * G::SLAB_A; };
  auto slabB = [&](int buf) { return lds + 2 * G::SLAB_A + buf * G::SLAB_B; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  // wave = (wk * WGM + wm) * WGN + wn; wk takes MFMA steps wk * SPW .. of each k-step
  // (KS = 1: the index arithmetic of the unsplit blocks, unchanged)
  const int wk = KS == 1 ? 0 : wave / (G::WGM * G::WGN);
  const int wmn = KS == 1 ? wave : wave - wk * (G::WGM * G::WGN);
  const int wm = (KS == 1 ? wave : wmn) / G::WGN, wn = (KS == 1 ? wave : wmn) % G::WGN;
  // within an XCD's run of tiles, walk groups of GM token blocks along N
  constexpr int GM = 4;
  // SPLIT: the XCD's run covers consecutive tiles of one split (one k-range),
  // which share the activation columns of that range
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int ntiles = SPLIT ? (int)(gridDim.x / splits) : (int)gridDim.x;
  const int split = SPLIT ? lin / ntiles : 0;
  const int tile = lin - split * ntiles;
  const int per = SPLIT ? (Kt + splits - 1) / splits : Kt;
  const int kt0 = split * per;                // first k-step of this workgroup
  const int nk = min(per, Kt - kt0);          // k-steps (>= 1: the host sizes the splits)
  const int tiles_m = ntiles / tiles_n;
  const int group = tile / (GM * tiles_n), within = tile - group * GM * tiles_n;
  const int gm = min(GM, tiles_m - group * GM);  // token blocks in this group
  const int tm = group * GM + within % gm, tn = within / gm;
  const int m0 = tm * BM, nt0 = tn * (BN / kTileN);  // first token, first 16-row weight tile
  const int r32 = lane & 31, g2 = lane >> 5;

  v16i acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][j][e] = 0;

  // activation pieces this thread moves: slot s = p*NT + tid holds piece
  // (s & 15) ^ (row & 15) of slab row s >> 4; rows past M read row M-1
  const int8_t* asrc[G::PA];
#pragma unroll
  for (int p = 0; p < G::PA; ++p) {
    const int s = p * G::NT + tid, row = s >> 4;
    asrc[p] = q + (int64_t)min(m0 + row, M - 1) * ldq + (((s & 15) ^ (row & 15)) * 16);
  }
  // weight pieces this thread moves: piece c = p*NT + tid is lane c % 64's
  // piece of local tile c / 64 (T2: the lane's 16 bytes; B1: the 8-byte half
  // of them this k-step reads); tiles past Nt read the last tile.  KtW is the
  // number of weight tiles per 16-row block (1 KB each).
  const BT* bsrc[G::PB];
#pragma unroll
  for (int p = 0; p < G::PB; ++p) {
    const int c = p * G::NT + tid;
    bsrc[p] = reinterpret_cast<const BT*>(packed + (int64_t)min(nt0 + (c >> 6), Nt - 1) * KtW * kTileBytes) +
              (FMT ? 2 * (c & 63) : (c & 63));
  }
  // this lane's weight chunks in the LDS slab: block j, chunk h
  int boff[NB][2];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lt = (wn * G::WN + 32 * j + r32) >> 4;  // local 16-row tile
      boff[j][h] = lt * G::TB + (16 * (2 * h + g2) + (r32 & 15)) * G::BP;
    }
  // LDS rows of this lane's activation operands; the swizzle term only
  // depends on r32 because every block starts on a multiple of 16 rows
  const int arow0 = wm * G::WM + r32;

  u4 aring[D][G::PA];
  BT bring[D][G::PB];
  auto load = [&](int u, int kt) {
#pragma unroll
    for (int p = 0; p < G::PA; ++p) aring[u][p] = *reinterpret_cast<const u4*>(asrc[p] + (int64_t)kt * kTileK);
#pragma unroll
    for (int p = 0; p < G::PB; ++p)
      bring[u][p] = FMT ? bsrc[p][(int64_t)(kt >> 1) * (kTileBytes / 8) + (kt & 1)] : bsrc[p][(int64_t)kt * 64];
  };
  auto stage_piece = [&](int u, int buf, int i) {  // i in [0, PA + PB)
    if (i < G::PA)
      *reinterpret_cast<u4*>(slabA(buf) + (i * G::NT + tid) * 16) = aring[u][i];
    else
      *reinterpret_cast<BT*>(slabB(buf) + ((i - G::PA) * G::NT + tid) * G::BP) = bring[u][i - G::PA];
  };
  // MFMA operand of step st from this lane's chunk pair
  auto expand = [&](const BT (&ch)[2], int st) -> v4i {
    if constexpr (FMT != 0) {
      const uint2 c = ch[st & 1];
      const uint32_t dw = (st >> 2) ? c.y : c.x;
      return b1_bytes((dw >> (16 * ((st >> 1) & 1))) & 0xFFFFu);
    } else {
      return t2_field(ch[st & 1], st >> 1);
    }
  };
  auto read_a = [&](v4i (&a)[MB], int buf, int s_) {
    const int c = 2 * s_ + g2;  // 16-byte piece: columns 32s + 16g
    const int off = (arow0 * 16 + (c ^ (r32 & 15))) * 16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const v4i*>(slabA(buf) + off + mb * 32 * kTileK);
  };

  // One k-step: 8 MFMA steps s = 2f + h, software-pipelined; the next
  // k-step's pieces are written to the other LDS half along the way.
  // (KS = 2: each half of the workgroup takes 4 of the 8 steps; the step
  // index must stay a compile-time constant, so the half is dispatched once)
  auto compute_half = [&](int buf, bool stage_next, int unext, auto half) {
    constexpr int SPW = G::SPW, ST0 = decltype(half)::value * SPW;
    BT wch[NB][2];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) wch[j][h] = *reinterpret_cast<const BT*>(slabB(buf) + boff[j][h]);
    v4i a[2][MB];
    v4i b[2][NB];
    read_a(a[0], buf, ST0);
#pragma unroll
    for (int j = 0; j < NB; ++j) b[0][j] = expand(wch[j], ST0);
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int st = ST0 + u, cur = u & 1, nx = cur ^ 1;
      if (u + 1 < SPW) {
        read_a(a[nx], buf, st + 1);
#pragma unroll
        for (int j = 0; j < NB; ++j) b[nx][j] = expand(wch[j], st + 1);
      }
      if (stage_next) {
#pragma unroll
        for (int i = u * (G::PA + G::PB) / SPW; i < (u + 1) * (G::PA + G::PB) / SPW; ++i)
          stage_piece(unext, buf ^ 1, i);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][j] = mfma32(a[cur][mb], b[cur][j], acc[mb][j]);
    }
  };
  auto compute = [&](int buf, bool stage_next, int unext) {
    if (KS == 1 || wk == 0)
      compute_half(buf, stage_next, unext, std::integral_constant<int, 0>{});
    else
      compute_half(buf, stage_next, unext, std::integral_constant<int, KS == 1 ? 0 : 1>{});
  };

  // LDS self-test builds: poison both halves before the first stage, and each
  // half again (this thread's own staging slots, so in program order before
  // its next data) once the barrier after its k-step has passed
  if constexpr (kLdsPoison) {
    lds_poison(lds, G::LDS);
    __syncthreads();
  }
  auto repoison = [&](int buf) {
    if constexpr (kLdsPoison) {
#pragma unroll
      for (int i = 0; i < G::PA; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          reinterpret_cast<uint32_t*>(slabA(buf) + (i * G::NT + tid) * 16)[w] = kLdsPoisonWord;
#pragma unroll
      for (int i = 0; i < G::PB; ++i)
#pragma unroll
        for (int w = 0; w < G::BP / 4; ++w)
          reinterpret_cast<uint32_t*>(slabB(buf) + (i * G::NT + tid) * G::BP)[w] = kLdsPoisonWord;
    }
  };

  // prologue: k-steps 0 .. D-1 requested (indices past the end re-read the
  // last k-step, in bounds, never used); k-step 0 into LDS half 0
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, kt0 + min(u, nk - 1));
#pragma unroll
  for (int i = 0; i < G::PA + G::PB; ++i) stage_piece(0, 0, i);
  __syncthreads();

  // full rounds of the ring, free of branches so the waits stay partial
  int k0 = 0;
  for (; k0 + D < nk; k0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int kt = k0 + u;
      load(u, kt0 + min(kt + D, nk - 1));  // slot u (k-step kt) went to LDS during the previous k-step
      compute(kt & 1, true, (u + 1) % D);
      __syncthreads();
      repoison(kt & 1);
    }
  }
  // the last 1..D k-steps (already requested)
#pragma unroll
  for (int u = 0; u < D; ++u) {
    const int kt = k0 + u;
    if (kt < nk) {  // uniform
      compute(kt & 1, kt + 1 < nk, (u + 1) % D);
      __syncthreads();
      repoison(kt & 1);
    }
  }

  const int n_wave = nt0 * kTileN + wn * G::WN;
  if constexpr (SPLIT) {
    // raw sums of this k-range into slice `split` of the workspace
    int32_t* slice = part + (int64_t)split * M * N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * G::WM + mb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int n = n_wave + 32 * j + r32;
          if (n < N) slice[(int64_t)m * N + n] = acc[mb][j][e];
        }
      }
    return;
  }
  // The per-row scales of the block go through LDS (the slabs are free: the
  // last k-step ended with a barrier), loaded once before any output store:
  // a global load between the stores would wait for every store issued
  // before it (vmcnt retires in order).
  if constexpr (kLdsPoison) {
    lds_poison(lds, G::LDS);
    __syncthreads();
  }
  float* s_ds = reinterpret_cast<float*>(lds);
  int* s_rs = reinterpret_cast<int*>(lds + BM * 4);
  const float bt = *beta;
  if (tid < BM) {
    s_ds[tid] = ds[min(m0 + tid, M - 1)];
    if constexpr (FMT != 0) s_rs[tid] = rowsum[min(m0 + tid, M - 1)];
  }
  __syncthreads();
  if constexpr (KS == 2) {
    // the second half of the workgroup hands its sums to the first through
    // LDS (behind the row scales; the slabs are free) and is done
    constexpr int PW = G::WGM * G::WGN * 64;  // lanes of one half
    static_assert(1024 + MB * NB * 16 * PW * 4 <= G::LDS && BM * 8 <= 1024, "LDS of the k-split exchange");
    int* xch = reinterpret_cast<int*>(lds + 1024);
    const int slot = wmn * 64 + lane;
    if (wk == 1) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) xch[((mb * NB + j) * 16 + e) * PW + slot] = acc[mb][j][e];
    }
    __syncthreads();
    if (wk == 1) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][j][e] += xch[((mb * NB + j) * 16 + e) * PW + slot];
  }
  // this lane's row scales, all read before the first store
  float scale[MB][16];
  int rsv[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = wm * G::WM + mb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
      scale[mb][e] = s_ds[r] * bt;
      rsv[mb][e] = FMT ? s_rs[r] : 0;
    }
  // the output type is dispatched once, outside the store loops
  auto emit = [&](auto ytype) {
    constexpr int YD = decltype(ytype)::value;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * G::WM + mb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int n = n_wave + 32 * j + r32;
          // B1: sum q * (2 b - 1) = 2 sum q * b - rowsum, scaled like the T2 sums (64 t)
          const int v = FMT ? (2 * acc[mb][j][e] - rsv[mb][e]) * 64 : acc[mb][j][e];
          if (n < N) store_out_t<YD>(y, (int64_t)m * N + n, v, scale[mb][e]);
        }
      }
  };
  switch (y_dtype) {
    case BITLINEAR_I32: emit(std::integral_constant<int, BITLINEAR_I32>{}); break;
    case BITLINEAR_F32: emit(std::integral_constant<int, BITLINEAR_F32>{}); break;
    case BITLINEAR_F32_ADD: emit(std::integral_constant<int, BITLINEAR_F32_ADD>{}); break;
    default: emit(std::integral_constant<int, BITLINEAR_BF16>{}); break;
  }
}

// Sum of the S workspace slices and the dequantization of the unsplit
// epilogue (the same expressions), one output element per thread; the slices
// are zeroed again, so the workspace leaves the call as it came in.
template <int FMT>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(int32_t* __restrict__ part, int S, int M, int N,
                                                          const float* __restrict__ ds,
                                                          const int32_t* __restrict__ rowsum,
                                                          const float* __restrict__ beta, void* __restrict__ y,
                                                          int y_dtype) {
  const int64_t mn = (int64_t)M * N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  int acc = 0;
  for (int sp = 0; sp < S; ++sp) {
    int32_t* p = part + sp * mn + i;
    acc += *p;
    *p = 0;
  }
  const int m = (int)(i / N);
  const float scale = ds[m] * *beta;
  const int v = FMT ? (2 * acc - rowsum[m]) * 64 : acc;
  store_out(y, y_dtype, i, v, scale);
}

template <int BM, int BN, int D, int FMT, bool SPLIT = false, int KS = 1>
hipError_t launch_tile(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M, int64_t K,
                       const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype, hipStream_t s,
                       int splits = 1, int32_t* part = nullptr) {
  using G = GemmTile<BM, BN, FMT, KS>;
  static LdsLimit lim;
  const hipError_t attr =
      ensure_lds_limit(lim, reinterpret_cast<const void*>(&gemm_t2_kernel<BM, BN, D, FMT, SPLIT, KS>), G::LDS);
  if (attr != hipSuccess) return attr;
  const int Nt = (int)ceil_div(N, kTileN), Kt = (int)ceil_div(K, kTileK);
  const int KtW = (int)ceil_div(K, FMT ? kTileKB1 : kTileK);
  const int tiles_n = (int)ceil_div(N, BN), tiles_m = (int)ceil_div(M, BM);
  hipLaunchKernelGGL((gemm_t2_kernel<BM, BN, D, FMT, SPLIT, KS>), dim3((unsigned)(tiles_m * tiles_n * splits)),
                     dim3(G::NT), G::LDS, s, q, ldq, ds, rowsum, (int)M, packed, beta, (int)N, Nt, Kt, KtW, tiles_n,
                     y, y_dtype, splits, part);
  if (!SPLIT) return hipGetLastError();
  hipLaunchKernelGGL((gemm_reduce_kernel<FMT>), dim3((unsigned)ceil_div(M * N, 256)), dim3(256), 0, s, part, splits,
                     (int)M, (int)N, ds, rowsum, beta, y, y_dtype);
  return hipGetLastError();
}

// Up to 64 tokens: 64 x 128 blocks, and k split across workgroups while the
// blocks alone leave at least half of the compute units idle (S whole
// multiples of the block count up to one workgroup per unit, each split
// keeping at least 4 k-steps).  Returns the number of splits; every split is
// non-empty.
constexpr int kMidM = 64, kMidN = 128, kSmallM = 32, kSmallN = 256, kMidGrid = 256, kMidMinSteps = 4;
int mid_splits(int64_t M, int64_t N, int64_t K, int bm, int bn) {
  const int64_t tiles = ceil_div(M, bm) * ceil_div(N, bn), Kt = ceil_div(K, kTileK);
  int64_t S = kMidGrid / tiles;
  if (S > Kt / kMidMinSteps) S = Kt / kMidMinSteps;
  if (S < 2) return 1;
  const int64_t per = ceil_div(Kt, S);
  return (int)ceil_div(Kt, per);
}
// Up to 32 tokens, when the 32 x 256 blocks would split k across workgroups
// but 32 x 128 blocks alone occupy at least half of the compute units (N of
// 16384 and more): 32 x 128 blocks with k split inside the workgroup.
constexpr int kSmallKsN = 128;
bool small_ks(int64_t M, int64_t N, int64_t K) {
  return M <= kSmallM && mid_splits(M, N, K, kSmallM, kSmallN) > 1 &&
         ceil_div(M, kSmallM) * ceil_div(N, kSmallKsN) * 2 >= kMidGrid;
}
int mid_splits(int64_t M, int64_t N, int64_t K) {
  if (small_ks(M, N, K)) return 1;
  return M <= kSmallM ? mid_splits(M, N, K, kSmallM, kSmallN) : mid_splits(M, N, K, kMidM, kMidN);
}

template <int BM, int BN, int FMT>
hipError_t launch_mid(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M, int64_t K,
                      const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype, hipStream_t s,
                      void* ws) {
  const int S = mid_splits(M, N, K, BM, BN);
  if (S > 1)
    return launch_tile<BM, BN, 3, FMT, true>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype, s, S,
                                             static_cast<int32_t*>(ws));
  return launch_tile<BM, BN, 3, FMT>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype, s);
}

template <int FMT>
hipError_t launch_fmt(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M, int64_t K,
                      const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype, hipStream_t s,
                      void* ws = nullptr) {
  if constexpr (FMT == 0) {
    if (small_ks(M, N, K))
      return launch_tile<kSmallM, kSmallKsN, 3, FMT, false, 2>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype,
                                                               s);
    if (M <= kSmallM)
      return launch_mid<kSmallM, kSmallN, FMT>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype, s, ws);
    if (M <= kMidM) return launch_mid<kMidM, kMidN, FMT>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype, s, ws);
  }
  // 128 x 256 blocks when that still gives a few hundred workgroups,
  // 128 x 128 otherwise
  const int64_t big = ceil_div(M, 128) * ceil_div(N, 256);
  if (big >= 384) return launch_tile<128, 256, 2, FMT>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype, s);
  return launch_tile<128, 128, 2, FMT>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype, s);
}

}  // namespace

int64_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M > kMidM) return 0;
  const int S = mid_splits(M, N, K);
  return S > 1 ? (int64_t)S * M * N * 4 : 0;
}

hipError_t launch_gemm_t2(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y,
                          int y_dtype, void* ws, hipStream_t s) {
  return launch_fmt<0>(q, ldq, ds, nullptr, M, K, packed, beta, N, y, y_dtype, s, ws);
}

hipError_t launch_gemm_b1(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype, hipStream_t s) {
  return launch_fmt<1>(q, ldq, ds, rowsum, M, K, packed, beta, N, y, y_dtype, s);
}

}  // namespace bl
