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
// for the three products; only the operand loaders differ.  A workgroup owns
// a T x T block of C: T = 256 with 8 waves (2 x 4, each 128 x 64) when the
// grid still covers most compute units, else T = 128 with 4 waves (2 x 2,
// each 64 x 64); waves compute 32 x 32 tiles with v_mfma_f32_32x32x16_bf16
// (lane l holds A[l % 32][8 (l / 32) + j] and B[8 (l / 32) + j][l % 32],
// j < 8).  The larger block halves the operand bytes per MFMA through L1 and
// LDS writes.  r advances in stages of 64:
//   * each thread moves 4 16-byte pieces of each operand per stage; they are
//     requested two stages ahead into a register ring and written into the
//     free half of double-buffered LDS tiles between the MFMAs of the stage
//     before, so the global-load latency is covered by two stages of work;
//   * sources whose rows run along the output index with r contiguous (x and
//     dy in the forward and dx products, t in the forward) are stored as
//     [row][r] and read with one 16-byte LDS read per operand;
//   * sources whose rows run along r (t in dx, dy and x in dw) are stored as
//     [r][row], still as 16-byte pieces, and read with two transposing LDS
//     reads (ds_read_b64_tr_b16: within 16 lanes, lane i receives element e
//     from the 8-byte address of lane 4 e + i / 4, at offset i % 4; pointing
//     lane j at row r0 + j / 4, column c0 + 4 (j % 4) gives lane i rows
//     r0 .. r0 + 3 of column c0 + i).
// When every bf16 row is a whole number of 16-byte pieces (row length a
// multiple of 8, 16-byte aligned base) the loads are clamped into the matrix
// and zeroed by a select, without branches, so the waits for a stage stay
// partial; other shapes take an element-wise loader.
//
// The ternary operands come straight from the 2-bit tiles: a piece of 8
// codes (n, k .. k + 7) is the field (k % 256) / 64 of bytes 8 ((k % 16) / 8)
// .. + 7 of tile lane 16 ((k % 64) / 16) + n % 16; two codes at a time become
// bf16 {-1, 0, +1} through one byte permute over constant tables.
#include "bl_internal.h"

namespace bl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool BIG>
struct TrainTile {
  static constexpr int T = BIG ? 256 : 128;        // block of C is T x T
  static constexpr int TR = BIG ? 32 : 64;         // stage of r (16 MFMAs per wave either way)
  static constexpr int PITCH = TR + 8;             // bf16 per [row][r] LDS row
  static constexpr int NT = BIG ? 512 : 256;       // threads per workgroup
  static constexpr int WQN = NT / 128;             // waves along Q (2 along P)
  static constexpr int WP = T / 2, WQ = T / WQN;   // per-wave block
  static constexpr int MI = WP / 32, NJ = WQ / 32; // 32 x 32 tiles per wave
  static constexpr int PPD = TR / 8;               // 16-byte pieces per [row][r] row
  static constexpr int PPR = T / 8;                // 16-byte pieces per [r][row] row
  // bf16 per [r][row] LDS row: T + 32, i.e. 16 banks mod 64.  A transposing
  // read serves 32 lanes per LDS cycle: two groups of 16 lanes, 8 banks
  // apart, each reading 8 banks in each of 4 consecutive rows; with a row
  // stride of 16 banks (mod 64) the 2 x 4 pieces fill the 64 banks once.
  static constexpr int PITCH_T = T + 32;
  static constexpr int OPND = T * PITCH > TR * PITCH_T ? T * PITCH : TR * PITCH_T;  // bf16 per operand tile
  static constexpr int LDS = 2 * 2 * OPND * 2;     // [buffer][A, B]
  static constexpr int NP = T * TR / 8 / NT;       // pieces per thread, operand and stage
  static_assert(NP == TR / 16, "one piece of each operand is stored per 16-wide MFMA step");
};

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

// bf16 bits of the codes in bytes 0 and 2 of y (2-bit two's complement t):
// the permute picks the low byte (0x80 unless t = 0) and the high byte (0x3F
// or 0xBF) of each value from constant tables indexed by the code.
__device__ inline uint32_t t2_pair(uint32_t y) {
  const uint32_t sel = y * 0x0101u + 0x00040004u;  // bytes: c0 + 4, c0, c1 + 4, c1
  return __builtin_amdgcn_perm(0x80008000u, 0xBF003F00u, sel);
}

// Field i of 8 packed bytes as 8 bf16 values (byte j -> value j).
__device__ inline u4 t2_decode(const uint2 w, int i) {
  u4 out;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t x = ((d ? w.y : w.x) >> (2 * i)) & 0x03030303u;
    out[2 * d] = t2_pair(__builtin_amdgcn_perm(x, x, 0x0c010c00u));
    out[2 * d + 1] = t2_pair(__builtin_amdgcn_perm(x, x, 0x0c030c02u));
  }
  return out;
}

// Eight ternary codes of row n, columns k .. k + 7 (k % 8 == 0) as bf16 bits;
// zero past the rows or tiles of t (the padding codes are 0 anyway).  The load
// is clamped into the tiles, so no branch is needed.
__device__ inline u4 t2_piece(const TrainArgs& a, int n, int k) {
  const int kmax = a.Kt * kTileK;
  const bool in = n < a.N && k < kmax;
  n = min(n, a.N - 1);
  k = min(k, kmax - 8);
  const int kb = k >> 8, c = k & 255;
  const int i = c >> 6, L = 16 * ((c & 63) >> 4) + (n & 15), h = (c & 15) >> 3;
  const uint2 w = *reinterpret_cast<const uint2*>(a.packed + ((int64_t)(n >> 4) * a.Kt + kb) * kTileBytes + 16 * L + 8 * h);
  const u4 v = t2_decode(w, i);
  return in ? v : u4{0u, 0u, 0u, 0u};
}

// Eight bf16 of row `row`, columns col .. col + 7 of a row-major source with
// `rows` rows and `cols` columns (row length ld); zero outside.  ALIGNED: ld
// == cols is a multiple of 8 and the base is 16-byte aligned.
template <bool ALIGNED>
__device__ inline u4 row_piece(const uint16_t* src, int ld, int rows, int cols, int row, int col) {
  if constexpr (ALIGNED) {
    const bool in = row < rows && col < cols;
    const u4 v = *reinterpret_cast<const u4*>(src + (int64_t)min(row, rows - 1) * ld + min(col, cols - 8));
    return in ? v : u4{0u, 0u, 0u, 0u};
  } else {
    if (row >= rows || col >= cols) return u4{0u, 0u, 0u, 0u};
    const uint16_t* p = src + (int64_t)row * ld + col;
    u4 out = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 8 && col + j < cols; ++j) out[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
    return out;
  }
}

// MFMA operand (8 bf16) of this lane from a [row][r] tile: rows row0 + l % 32,
// r = r0 + 8 (l / 32) .. + 7.
template <int PITCH>
__device__ inline bf16x8 read_direct(const uint16_t* t, int row0, int r0, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + (row0 + (lane & 31)) * PITCH + r0 + 8 * (lane >> 5));
}

// The same operand from an [r][row] tile with two transposing reads.
template <int PITCH_T>
__device__ inline bf16x8 read_transposed(const uint16_t* t, int row0, int r0, int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int col = row0 + 16 * (grp & 1) + 4 * (i & 3);
  const int r = r0 + 8 * (grp >> 1) + (i >> 2);
  typedef __attribute__((address_space(3))) s16x4 lds_v4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(t + r * PITCH_T + col));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(t + (r + 4) * PITCH_T + col));
  // one whole-vector shuffle: rebuilding the operand element by element from
  // the two reads has been folded into a splat of element 0 by the compiler
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int MODE, bool ALIGNED, bool BIG>
__global__ __launch_bounds__(TrainTile<BIG>::NT) void train_gemm_kernel(const TrainArgs a) {
  using G = TrainTile<BIG>;
  constexpr int T = G::T, NT = G::NT, NP = G::NP, OPND = G::OPND, PPR = G::PPR, MI = G::MI, NJ = G::NJ;
  constexpr int TR = G::TR, PITCH = G::PITCH, PPD = G::PPD;
  // A (and B) is stored transposed, as [r][row], when its source rows run along r
  constexpr bool AT = MODE == DW, BT = MODE != FWD;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [buffer][A, B][OPND]
  if constexpr (kLdsPoison) {  // LDS self-test builds
    lds_poison(lds, G::LDS);
    __syncthreads();
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave / G::WQN, wq = wave % G::WQN;
  // the XCD's contiguous run of tiles, walked in groups of 4 row blocks of C
  // along Q (they share their A rows and B columns in that XCD's L2)
  constexpr int GM = 4;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int tiles_p = (int)(gridDim.x / a.tiles_q);
  const int group = tile / (GM * a.tiles_q), within = tile - group * GM * a.tiles_q;
  const int gm = min(GM, tiles_p - group * GM);
  const int tp = group * GM + within % gm, tq = within / gm;
  const int p0 = tp * T, q0 = tq * T;
  const int l32 = lane & 31, g = lane >> 5;

  // Pieces of a source row-major along r: piece c -> row c / PPD, r 8 (c % PPD).
  // Pieces of a source whose rows run along r: piece c -> r c / PPR, row
  // (P or Q index) 8 (c % PPR).
  auto load = [&](u4 (&pa)[NP], u4 (&pb)[NP], int r0) {
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      const int c = h * NT + tid;
      if constexpr (MODE == DW) {
        pa[h] = row_piece<ALIGNED>(a.a, a.lda, a.R, a.P, r0 + c / PPR, p0 + 8 * (c % PPR));  // dy[m][n], n along P
        pb[h] = row_piece<ALIGNED>(a.b, a.ldb, a.R, a.Q, r0 + c / PPR, q0 + 8 * (c % PPR));  // x[m][k], k along Q
      } else {
        pa[h] = row_piece<ALIGNED>(a.a, a.lda, a.P, a.R, p0 + c / PPD, r0 + 8 * (c % PPD));   // x or dy rows
        if constexpr (MODE == FWD)
          pb[h] = t2_piece(a, q0 + c / PPD, r0 + 8 * (c % PPD));                              // t[n][k], k along r
        else
          pb[h] = t2_piece(a, r0 + c / PPR, q0 + 8 * (c % PPR));                             // t[n][k], n along r
      }
    }
  };
  // LDS slot of piece c: the same pieces the loaders fetch
  auto slot = [](bool tr, int c) { return tr ? (c / PPR) * G::PITCH_T + 8 * (c % PPR) : (c / PPD) * PITCH + 8 * (c % PPD); };
  auto store_piece = [&](int buf, const u4 (&pa)[NP], const u4 (&pb)[NP], int h) {
    const int c = h * NT + tid;
    *reinterpret_cast<u4*>(lds + (2 * buf) * OPND + slot(AT, c)) = pa[h];
    *reinterpret_cast<u4*>(lds + (2 * buf + 1) * OPND + slot(BT, c)) = pb[h];
  };
  auto read_ops = [&](bf16x8 (&av)[MI], bf16x8 (&bv)[NJ], const uint16_t* A, const uint16_t* B, int ks) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
      av[i] = AT ? read_transposed<G::PITCH_T>(A, wp * G::WP + 32 * i, 16 * ks, lane)
                 : read_direct<PITCH>(A, wp * G::WP + 32 * i, 16 * ks, lane);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      bv[j] = BT ? read_transposed<G::PITCH_T>(B, wq * G::WQ + 32 * j, 16 * ks, lane)
                 : read_direct<PITCH>(B, wq * G::WQ + 32 * j, 16 * ks, lane);
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // One stage from LDS half buf; the pieces (na, nb) of a later stage go to
  // the other half, one of each per 16-wide step, between the MFMAs.
  auto compute = [&](int buf, const u4 (&na)[NP], const u4 (&nb)[NP]) {
    const uint16_t* A = lds + (2 * buf) * OPND;
    const uint16_t* B = lds + (2 * buf + 1) * OPND;
    // the small block reads the next step's operands during the current
    // step's MFMAs; the large one has no registers to spare for that
    constexpr int OB = BIG ? 1 : 2;
    bf16x8 av[OB][MI], bv[OB][NJ];
    read_ops(av[0], bv[0], A, B, 0);
#pragma unroll
    for (int ks = 0; ks < TR / 16; ++ks) {
      const int cur = OB == 2 ? (ks & 1) : 0;
      if (OB == 2 && ks + 1 < TR / 16) read_ops(av[(ks + 1) % OB], bv[(ks + 1) % OB], A, B, ks + 1);
      if (OB == 1 && ks > 0) read_ops(av[0], bv[0], A, B, ks);
      store_piece(buf ^ 1, na, nb, ks);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][i], bv[cur][j], acc[i][j], 0, 0, 0);
    }
  };

  // ring of two stages in registers; requests past the last stage re-read it
  // (in bounds) and their pieces are never read from LDS
  const int steps = (a.R + TR - 1) / TR;
  auto rs = [&](int s) { return min(s, steps - 1) * TR; };
  u4 ra0[NP], rb0[NP], ra1[NP], rb1[NP];
  load(ra0, rb0, rs(0));
  load(ra1, rb1, rs(1));
#pragma unroll
  for (int h = 0; h < NP; ++h) store_piece(0, ra0, rb0, h);
  __syncthreads();
  int s = 0;
  for (; s + 2 <= steps; s += 2) {
    load(ra0, rb0, rs(s + 2));  // stage s went to LDS half 0 before
    compute(0, ra1, rb1);       // stage s; stage s + 1 into half 1
    __syncthreads();
    load(ra1, rb1, rs(s + 3));
    compute(1, ra0, rb0);       // stage s + 1; stage s + 2 into half 0
    __syncthreads();
  }
  if (s < steps) compute(0, ra1, rb1);  // the last stage (its copy into half 1 is never read)

  const float scale = MODE == DW ? 1.0f : *a.beta;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int p = p0 + wp * G::WP + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
      if (p >= a.P) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = q0 + wq * G::WQ + 32 * j + l32;
        if (q < a.Q) a.c[(int64_t)p * a.Q + q] = __fmul_rn(acc[i][j][e], scale);
      }
    }
}

template <int MODE, bool ALIGNED, bool BIG>
hipError_t launch_tile(TrainArgs a, hipStream_t s) {
  using G = TrainTile<BIG>;
  static LdsLimit lim;
  const hipError_t attr = ensure_lds_limit(lim, reinterpret_cast<const void*>(&train_gemm_kernel<MODE, ALIGNED, BIG>),
                                           G::LDS);
  if (attr != hipSuccess) return attr;
  a.tiles_q = (a.Q + G::T - 1) / G::T;
  const int tiles_p = (a.P + G::T - 1) / G::T;
  hipLaunchKernelGGL((train_gemm_kernel<MODE, ALIGNED, BIG>), dim3((unsigned)(tiles_p * a.tiles_q)), dim3(G::NT),
                     G::LDS, s, a);
  return hipGetLastError();
}

// Block size for aligned operands, from rounds over the 256 compute units:
// one 256 x 256 block per unit and round, or two 128 x 128 blocks per unit
// and round; a 256-block does the work of four 128-blocks about 1.25 times
// as efficiently (measured), so it wins when 4 / 1.25 * rounds(256) < 2 *
// rounds(128).  Unaligned operands take the 128 x 128 kernel.
constexpr int64_t kCUs = 256;
template <int MODE>
hipError_t launch(const TrainArgs& a, bool aligned, hipStream_t s) {
  if (!aligned) return launch_tile<MODE, false, false>(a, s);
  const int64_t r256 = ceil_div(ceil_div(a.P, 256) * ceil_div(a.Q, 256), kCUs);
  const int64_t r128 = ceil_div(ceil_div(a.P, 128) * ceil_div(a.Q, 128), 2 * kCUs);
  if (16 * r256 < 10 * r128) return launch_tile<MODE, true, true>(a, s);
  return launch_tile<MODE, true, false>(a, s);
}

// bf16 rows of `len` values starting at p are whole, aligned 16-byte pieces
bool pieces(const void* p, int64_t len) { return len % 8 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

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
  return launch<FWD>(a, pieces(x, K), s);
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
  return launch<DX>(a, pieces(dy, N), s);
}

hipError_t launch_train_dw(const uint16_t* dy, const uint16_t* x, int64_t M, int64_t N, int64_t K, float* dw,
                           hipStream_t s) {
  TrainArgs a{};
  a.a = dy;
  a.b = x;
  a.c = dw;
  a.P = (int)N, a.Q = (int)K, a.R = (int)M;
  a.lda = (int)N, a.ldb = (int)K;
  return launch<DW>(a, pieces(dy, N) && pieces(x, K), s);
}

}  // namespace bl
