// Training step of a BitLinear with the straight-through estimator ("BitNet /
// Ternary / Binary - Les LLMs 1-bit", Apercu de l'entrainement d'un
// BitLinear): the forward multiplies by the quantized weights, the backward
// lets the gradient reach the latent weights unchanged.
//
//   forward   y [M][N] = beta * x . t^T        (x bf16 [M][K], t ternary [N][K])
//   input     dx[M][K] = beta * dy . t         (dy bf16 [M][N])
//   weight    dw[N][K] = dy^T . x
//
// One bf16 matrix-core kernel computes C[P][Q] = scale * sum_r A(p, r) B(q, r)
// for the three products; only the operand loaders differ.  A workgroup of
// 4 waves (2 x 2) owns a 128 x 128 block of C, each wave 64 x 64 as 2 x 2
// tiles of v_mfma_f32_32x32x16_bf16 (lane l holds A[l % 32][8 (l / 32) + j]
// and B[8 (l / 32) + j][l % 32], j < 8).  Per 32-wide step of r both operand
// tiles are staged in LDS in the orientation of their source, always as
// 16-byte pieces, and the next step's pieces are loaded into registers while
// the current step's MFMAs run:
//   * sources whose rows run along the output index with r contiguous (x and
//     dy in the forward and dx products, t in the forward) are stored as
//     [row][r] and read with one 16-byte LDS read per operand;
//   * sources whose rows run along r (t in dx, dy and x in dw) are stored as
//     [r][row] and read with two transposing LDS reads (ds_read_b64_tr_b16:
//     within 16 lanes, lane i receives element e from the 8-byte address of
//     lane 4 e + i / 4, at offset i % 4; pointing lane j at row r0 + j / 4,
//     column c0 + 4 (j % 4) gives lane i rows r0 .. r0 + 3 of column c0 + i).
// The ternary operands come straight from the 2-bit tiles: a piece of 8
// codes (n, k .. k + 7) is the field (k % 256) / 64 of bytes 8 ((k % 16) / 8)
// .. + 7 of tile lane 16 ((k % 64) / 16) + n % 16, widened to bf16 {-1, 0, +1}.
#include "bl_internal.h"

namespace bl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TP = 128, TQ = 128, TR = 32;  // block of C, step of r
constexpr int PITCH = TR + 8;               // bf16 per [row][r] LDS row (80 bytes)
constexpr int PITCH_T = TP + 8;             // bf16 per [r][row] LDS row (272 bytes)
constexpr int OPND = TP * PITCH > TR * PITCH_T ? TP * PITCH : TR * PITCH_T;  // bf16 per operand tile

enum TrainMode { FWD = 0, DX = 1, DW = 2 };

struct TrainArgs {
  const uint16_t* a;   // FWD: x [M][K]; DX: dy [M][N]; DW: dy [M][N]
  const uint16_t* b;   // DW: x [M][K]
  const uint8_t* packed;  // FWD, DX: 2-bit tiles of t [N][K]
  const float* beta;   // FWD, DX
  float* c;
  int P, Q, R;         // C is P x Q, contraction length R
  int lda, ldb;        // row lengths of a and b (elements)
  int Kt, N;           // tiles per 16-row block of t, rows of t
  int tiles_q;
};

// Eight ternary codes of row n, columns k .. k + 7 (k % 8 == 0) as bf16 bits;
// zero past the rows or tiles of t (the padding codes are 0 anyway).
__device__ inline u4 t2_piece(const TrainArgs& a, int n, int k) {
  if (n >= a.N || k >= a.Kt * kTileK) return u4{0u, 0u, 0u, 0u};
  const int kb = k >> 8, c = k & 255;
  const int i = c >> 6, L = 16 * ((c & 63) >> 4) + (n & 15), h = (c & 15) >> 3;
  const uint2 w = *reinterpret_cast<const uint2*>(a.packed + ((int64_t)(n >> 4) * a.Kt + kb) * kTileBytes + 16 * L + 8 * h);
  u4 out;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t word = d ? w.y : w.x;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint32_t pair = 0;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint32_t code = (word >> (8 * (2 * p + b) + 2 * i)) & 3u;  // 01 = +1, 11 = -1, 00 = 0
        const uint32_t v = (code & 1u) ? (0x3F80u | ((code & 2u) << 14)) : 0u;
        pair |= v << (16 * b);
      }
      out[2 * d + p] = pair;
    }
  }
  return out;
}

// Eight bf16 of row `row`, columns col .. col + 7 of a row-major source with
// `rows` rows and `cols` columns; zero outside.
__device__ inline u4 row_piece(const uint16_t* src, int ld, int rows, int cols, int row, int col) {
  if (row >= rows || col >= cols) return u4{0u, 0u, 0u, 0u};
  const uint16_t* p = src + (int64_t)row * ld + col;
  if (col + 8 <= cols && (reinterpret_cast<uintptr_t>(p) & 15) == 0) return *reinterpret_cast<const u4*>(p);
  u4 out = {0u, 0u, 0u, 0u};
  for (int j = 0; j < 8 && col + j < cols; ++j) out[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
  return out;
}

// MFMA operand (8 bf16) of this lane from a [row][r] tile: rows row0 + l % 32,
// r = r0 + 8 (l / 32) .. + 7.
__device__ inline bf16x8 read_direct(const uint16_t* t, int row0, int r0, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + (row0 + (lane & 31)) * PITCH + r0 + 8 * (lane >> 5));
}

// The same operand from an [r][row] tile with two transposing reads.
__device__ inline bf16x8 read_transposed(const uint16_t* t, int row0, int r0, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int col = row0 + 16 * (grp & 1) + 4 * (i & 3);
  const int r = r0 + 8 * (grp >> 1) + (i >> 2);
  typedef __attribute__((address_space(3))) s16x4 lds_v4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(t + r * PITCH_T + col));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(t + (r + 4) * PITCH_T + col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int MODE>
__global__ __launch_bounds__(256) void train_gemm_kernel(const TrainArgs a) {
  // A (and B) is stored transposed, as [r][row], when its source rows run along r
  constexpr bool AT = MODE == DW, BT = MODE != FWD;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][OPND];  // [buffer][A, B]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave >> 1, wq = wave & 1;
  const int tp = blockIdx.x / a.tiles_q, tq = blockIdx.x - tp * a.tiles_q;
  const int p0 = tp * TP, q0 = tq * TQ;
  const int l32 = lane & 31, g = lane >> 5;

  // Each thread moves two 8-value pieces of each operand per step.  Pieces
  // of a row-major source along r: piece c -> row c / 4, columns 8 (c % 4).
  // Pieces of a source whose rows run along r (transposed into LDS): piece c
  // -> source row (r) c / 16, columns (P or Q index) 8 (c % 16).
  u4 pa[2], pb[2];
  auto load = [&](int r0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * 256 + tid;
      if constexpr (MODE == DW) {
        pa[h] = row_piece(a.a, a.lda, a.R, a.P, r0 + (c >> 4), p0 + 8 * (c & 15));  // dy[m][n], n along P
        pb[h] = row_piece(a.b, a.ldb, a.R, a.Q, r0 + (c >> 4), q0 + 8 * (c & 15));  // x[m][k], k along Q
      } else {
        pa[h] = row_piece(a.a, a.lda, a.P, a.R, p0 + (c >> 2), r0 + 8 * (c & 3));   // x or dy rows
        if constexpr (MODE == FWD)
          pb[h] = t2_piece(a, q0 + (c >> 2), r0 + 8 * (c & 3));                     // t[n][k], k along r
        else
          pb[h] = t2_piece(a, r0 + (c >> 4), q0 + 8 * (c & 15));                    // t[n][k], n along r
      }
    }
  };
  // piece c of a [row][r] tile: row c / 4, r 8 (c % 4); of an [r][row] tile:
  // r c / 16, rows 8 (c % 16) -- the same pieces the loaders fetch
  auto slot = [](bool tr, int c) { return tr ? (c >> 4) * PITCH_T + 8 * (c & 15) : (c >> 2) * PITCH + 8 * (c & 3); };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * 256 + tid;
      *reinterpret_cast<u4*>(lds[buf][0] + slot(AT, c)) = pa[h];
      *reinterpret_cast<u4*>(lds[buf][1] + slot(BT, c)) = pb[h];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int steps = (a.R + TR - 1) / TR;
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < steps) load((s + 1) * TR);  // in flight during the MFMAs
    const uint16_t* A = lds[buf][0];
    const uint16_t* B = lds[buf][1];
#pragma unroll
    for (int ks = 0; ks < TR / 16; ++ks) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = AT ? read_transposed(A, wp * 64 + 32 * i, 16 * ks, lane) : read_direct(A, wp * 64 + 32 * i, 16 * ks, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = BT ? read_transposed(B, wq * 64 + 32 * j, 16 * ks, lane) : read_direct(B, wq * 64 + 32 * j, 16 * ks, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < steps) store(buf ^ 1);
    __syncthreads();
  }

  const float scale = MODE == DW ? 1.0f : *a.beta;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int p = p0 + wp * 64 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
      if (p >= a.P) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = q0 + wq * 64 + 32 * j + l32;
        if (q < a.Q) a.c[(int64_t)p * a.Q + q] = __fmul_rn(acc[i][j][e], scale);
      }
    }
}

template <int MODE>
hipError_t launch(const TrainArgs& a, hipStream_t s) {
  const int tiles_p = (a.P + TP - 1) / TP;
  hipLaunchKernelGGL((train_gemm_kernel<MODE>), dim3((unsigned)(tiles_p * a.tiles_q)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_train_forward(const uint16_t* x, int64_t M, int64_t K, const uint8_t* packed, const float* beta,
                                int64_t N, float* y, hipStream_t s) {
  TrainArgs a{};
  a.a = x;
  a.packed = packed;
  a.beta = beta;
  a.c = y;
  a.P = (int)M, a.Q = (int)N, a.R = (int)K;
  a.lda = (int)K;
  a.Kt = (int)ceil_div(K, kTileK), a.N = (int)N;
  a.tiles_q = (int)ceil_div(N, TQ);
  return launch<FWD>(a, s);
}

hipError_t launch_train_dx(const uint16_t* dy, int64_t M, int64_t N, const uint8_t* packed, const float* beta,
                           int64_t K, float* dx, hipStream_t s) {
  TrainArgs a{};
  a.a = dy;
  a.packed = packed;
  a.beta = beta;
  a.c = dx;
  a.P = (int)M, a.Q = (int)K, a.R = (int)N;
  a.lda = (int)N;
  a.Kt = (int)ceil_div(K, kTileK), a.N = (int)N;
  a.tiles_q = (int)ceil_div(K, TQ);
  return launch<DX>(a, s);
}

hipError_t launch_train_dw(const uint16_t* dy, const uint16_t* x, int64_t M, int64_t N, int64_t K, float* dw,
                           hipStream_t s) {
  TrainArgs a{};
  a.a = dy;
  a.b = x;
  a.c = dw;
  a.P = (int)N, a.Q = (int)K, a.R = (int)M;
  a.lda = (int)N, a.ldb = (int)K;
  a.tiles_q = (int)ceil_div(K, TQ);
  return launch<DW>(a, s);
}

}  // namespace bl
