// Decode-shaped ternary product (M <= 64 tokens) with fused dequantization,
// and its fused variant that also quantizes the activations.
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
// columns).  A workgroup owns NB consecutive 16-row output blocks; its waves
// split the k-tiles into contiguous ranges.  Per k-tile a wave reads 16 bytes
// per lane of each of its NB weight tiles (one coalesced 1 KB load each, kU
// k-tiles ahead of use), expands each 2-bit field into an MFMA operand and
// issues 4 * MB * NB MFMA 16x16x64 steps.  The waves add their partial sums
// with LDS atomics; wave 0 dequantizes and stores.  Wide plans (one token
// block, 1024..2048 output blocks) run one workgroup per compute unit over
// ceil(Nt / 256) blocks instead, with interleaved k-tiles (wave w takes w,
// w + waves, ...), so that the workgroup reads its tile range in address
// order; their int8 rows may use most of the unit's LDS.
//
// Activation operands (the int8 token rows) come from one of three places:
//   ALDS_Q  the workgroup copies the int8 rows into LDS once (16-byte loads,
//           rows padded by 16 bytes so the 16 token rows fall on different
//           banks) and reads its operands from there;
//   ALDS_X  fused quantization: the workgroup reads the bf16/fp32 rows, finds
//           each row's absmax and writes the int8 rows into LDS itself, with
//           the same arithmetic as the standalone quantizer ("Key
//           Technologies Enabling the BitNET Family", Advanced Quantization
//           Methodologies: per-token absmax 8-bit activations);
//   ALDS_XS the same for rows that are not whole 16-byte pieces (unaligned x
//           or K not a multiple of 8 bf16 / 4 fp32), element by element;
//   AGLOBAL the rows are too large for LDS: operands are 16-byte global loads
//           carried in the same ring as the weight tiles and reused over the
//           NB weight tiles of a k-tile.
// In every mode the first weight tiles are requested before the activations.
//
// One launch can serve several BitLinears that read the same activations
// (segments: e.g. the q, k and v projections of a decoder layer): the output
// groups of all segments form one grid, and each workgroup finds its segment
// from the group index.  A gated pair (gate and up projections of the same
// shape) runs with NB = 2, tile j = 0 from the gate and j = 1 from the up
// matrix at the same rows, and its epilogue writes h = ReLU(y_gate)^2 * y_up
// ("Key Technologies Enabling the BitNET Family", Architectural Innovations
// and Optimizations: squared ReLU in the feed-forward layers) instead of the
// two outputs.
//
// Binary weights (format B1, "BitNet / Ternary / Binary - Les LLMs 1-bit",
// TL;DR: every weight +1 or -1) use the same kernel with 16 x 512 tiles of
// one bit per weight: lane (n, g) of step s holds the 16 bits of columns
// 64 s + 16 g + j, expanded to bytes b in {0, 1} with one multiply per four
// bits; the matrix cores sum q * b and the epilogue takes 2 * sum - rowsum(q)
// = sum q * (2 b - 1), exact.
//
// Base-3 tiles (format B3, five ternary weights per byte) hold 16 x 320
// weights per 1 KB: byte i of lane (n, g) carries, in base 3, the codes
// c = t + 1 of columns 64 s + 16 g + i for the five steps s.  Digit s of four
// bytes at a time comes from exact 16-bit multiply-shift divisions by 3^s
// (two bytes per 16-bit half), the matrix cores sum q * c with c in {0, 1, 2},
// and the epilogue subtracts rowsum(q): sum q * (c - 1) = sum q * t.
//
// Tiny outputs with a long K (AGLOBAL only) also split K across workgroups:
// their sums meet in an int32 workspace through device-scope atomics and the
// last workgroup to arrive (a counter) dequantizes, stores y and zeroes the
// workspace again.
#include <algorithm>
#include <type_traits>

#include "bl_internal.h"

namespace bl {
namespace {

constexpr float kEpsX = 1e-5f;
// 16-byte activation pieces a thread of a fused launch loads before the
// weight prefetch and holds in registers until the weight loads are in flight.
constexpr int kXReg = 8;
constexpr int kLdsPad = 16;  // bytes added to each LDS activation row
// Residency of the LDS-staged plans: compute units, LDS per unit, and a bound
// on the kernel's static LDS (reduction buffer and row scales).
constexpr int64_t kResidentCUs = 256, kLdsPerCU = 160 * 1024, kGemvStaticLds = 4608;
enum AMode { AGLOBAL = 0, ALDS_Q = 1, ALDS_X = 2, ALDS_XS = 3 };

// k-tiles in flight per wave, chosen to keep the prefetch ring within the
// register budget (weights: 4 VGPRs per output block; activations in the
// ring only for AGLOBAL: 16 VGPRs per token block).
// MFMA steps per 1 KB weight tile: 4 (T2), 8 (B1), 5 (B3).
constexpr int tile_steps(int fmt) { return fmt == 1 ? 8 : (fmt == 2 ? 5 : 4); }
// Columns per weight tile: 256 (T2, 2 bits), 512 (B1, 1 bit), 320 (B3, 1.6 bits).
constexpr int tile_cols(int fmt) { return 64 * tile_steps(fmt); }

// Formats with more steps per tile carry more activation operands per tile.
// Wide plans (4 or more output blocks) keep one k-step of NB tiles in flight:
// measured on 28672 x 8192 (7 blocks), 12.6 us against 14.2 us with two.
constexpr int ring_depth(int mb, int nb, int amode, int fmt = 0) {
  return amode == AGLOBAL ? ((tile_steps(fmt) * mb + nb) * 4 <= 24 ? 4 : ((tile_steps(fmt) * mb + nb) * 4 <= 40 ? 2 : 1))
                          : (nb == 1 ? 8 : (nb == 2 ? 4 : (nb >= 4 ? 1 : 2)));
}
// Largest workgroup, in waves, for MB token blocks.
constexpr int max_waves(int mb) { return mb <= 2 ? 16 : 8; }
// The same for MB token blocks and NB output blocks: 4 or more output blocks
// with one token block are the wide plans, at most kWideWaves waves, which
// leaves each wave the register file of two waves per SIMD.
constexpr int kWideWaves = 8;
constexpr int max_waves(int mb, int nb) { return mb == 1 && nb >= 4 ? kWideWaves : max_waves(mb); }

int64_t lds_row(int64_t K, int fmt = 0) { return ceil_div(K, tile_cols(fmt)) * tile_cols(fmt) + kLdsPad; }

struct GemvPlan {
  int MB, NB;      // 16-row token blocks, 16-row output blocks per workgroup
  int Nt, Kt, Ng;  // output blocks, k-tiles, output groups (Nt / NB)
  int waves, SB;   // waves per workgroup, workgroups per output group
  int tps;         // k-tiles per wave
  int kint;        // 1: wave w takes k-tiles w, w + waves, ... (else a run of tps)
  int bigx;        // wide plan whose int8 rows exceed kXReg pieces per thread
  int amode;       // where activation operands come from
  int64_t lds_bytes;
  int64_t ws_acc_bytes, ws_bytes;
};

// Wide plans (one token block, 2-bit tiles, activation rows in LDS, a single
// matrix of kWideMinNt..kWideMaxNB * 256 output blocks): one workgroup per
// compute unit owns ceil(Nt / 256) consecutive output blocks, and its
// kWideWaves waves take interleaved k-tiles (wave w: w, w + 8, ...), so the
// workgroup sweeps its contiguous range of tiles in address order.  Measured
// on 28672 x 8192 (1792 blocks of 32 k-tiles): a plain read in this order
// takes 10.1 us against 11.2 us with 896 workgroups of two blocks (3.5 per
// unit) and per-wave k-runs.
constexpr int kWideMinNt = 1024, kWideMaxNB = 8;
// Int8 rows a wide plan may stage in LDS: one workgroup per compute unit
// leaves the unit's 160 KB to it, less the static reduction buffer (<= 10.5 KB).
constexpr int64_t kWideLdsBytes = 144 * 1024;

// A single matrix that wide plans cover with rows of lds bytes in LDS.
bool wide_shape(int64_t M, int64_t Nt, int64_t lds, int fmt, bool fuse) {
  return fmt == 0 && M >= 1 && M <= 16 && Nt >= kWideMinNt && Nt <= (int64_t)kWideMaxNB * kResidentCUs &&
         (fuse ? lds <= kDecodeLdsBytes : lds <= kWideLdsBytes);
}

// xpieces: 16-byte activation pieces of a fused launch whose rows are whole
// pieces (0 otherwise).  wide: a single matrix, so wide plans may be used.
GemvPlan make_plan(int64_t M, int64_t N, int64_t K, bool fuse, bool allow_split = true, int64_t xpieces = 0,
                   int fmt = 0, bool wide = false) {
  GemvPlan p{};
  p.MB = (int)ceil_div(M < 1 ? 1 : M, 16);
  p.Nt = (int)ceil_div(N, kTileN);
  p.Kt = (int)ceil_div(K, tile_cols(fmt));
  const int64_t lds = M * lds_row(K, fmt);
  p.amode = fuse ? ALDS_X : (lds <= kDecodeLdsBytes ? ALDS_Q : AGLOBAL);
  p.lds_bytes = p.amode == AGLOBAL ? 0 : lds;
  p.SB = 1;
  if (wide && wide_shape(M, p.Nt, lds, fmt, fuse)) {
    // fused: enough threads to hold the activation rows in registers, within
    // the wide instantiations' launch bound of kWideWaves waves (int8 rows
    // beyond the registers are copied to LDS by a loop instead)
    const int64_t need = fuse ? ceil_div(xpieces, (int64_t)kXReg * 64) : 1;
    if (need <= kWideWaves) {
      p.amode = fuse ? ALDS_X : ALDS_Q;
      p.lds_bytes = lds;
      p.NB = (int)ceil_div(p.Nt, kResidentCUs);
      p.Ng = (int)ceil_div(p.Nt, p.NB);
      const int waves = p.Kt < kWideWaves ? p.Kt : kWideWaves;
      p.waves = (int)(waves < need ? need : waves);
      p.tps = (int)ceil_div(p.Kt, p.waves);
      p.kint = 1;
      p.bigx = !fuse && xpieces > (int64_t)kXReg * 64 * p.waves;
      return p;
    }
  }
  // Output blocks per workgroup: each activation operand is reused over NB
  // weight tiles; N decides how many workgroups remain.  The LDS modes cap
  // MB * NB at 4 (4 KB reduction buffer next to the activation rows).
  // k-tiles per wave: long runs for one token block (the weight stream is the
  // only work), shorter ones once MFMA work grows with the token count.
  // Both rules are fitted to measurements on the 2B- and 100B-class shapes.
  if (p.MB == 1) {
    p.NB = p.Nt >= 384 ? 2 : 1;
  } else {
    p.NB = p.Nt >= 1024 ? 4 : (p.Nt >= 384 ? 2 : 1);
  }
  const int nb_cap = p.amode == AGLOBAL ? (p.MB > 2 ? 2 : 4) : (p.MB >= 3 ? 1 : 4 / p.MB);
  if (p.NB > nb_cap) p.NB = nb_cap;
  p.Ng = (int)ceil_div(p.Nt, p.NB);
  if (p.amode == ALDS_Q && p.Ng > kResidentCUs * (kLdsPerCU / (lds + kGemvStaticLds))) {
    // the staged rows would leave too few workgroups resident for one
    // round: read the operands from global memory instead (measured on
    // 6 x 8192 -> 28672 with two-block workgroups: 16.4 us against 21.2 us;
    // that shape now takes a wide plan, 14.1 us)
    p.amode = AGLOBAL;
    p.lds_bytes = 0;
    p.NB = p.NB > (p.MB > 2 ? 2 : 4) ? (p.MB > 2 ? 2 : 4) : p.NB;
    p.Ng = (int)ceil_div(p.Nt, p.NB);
  }
  const int maxw = max_waves(p.MB);
  // one token block with operands from global memory, many output groups and
  // 32 or more k-tiles (e.g. 8 tokens, K = 8192 at 2 bits): one wave streams
  // 32 k-tiles
  const int target =
      p.MB == 1 ? (p.Kt >= 32 ? (p.amode == AGLOBAL && p.Ng >= 512 ? 32 : 16) : 8) : 5;
  int waves = (int)ceil_div(p.Kt, target);
  if (p.MB == 1 && p.Ng < 512) {
    // about one workgroup per CU: keep all four SIMDs busy with whole
    // multiples of four waves (measured on the 2B- and 100B-class shapes)
    waves = p.Kt < 32 ? 4 : (int)ceil_div(waves, 4) * 4;
  }
  if (waves > maxw) waves = maxw;
  if (waves < 1) waves = 1;
  p.tps = (int)ceil_div(p.Kt, waves);
  p.waves = (int)ceil_div(p.Kt, p.tps);
  if (xpieces > 0 && p.amode != AGLOBAL) {
    // enough threads to hold the activation rows in registers; the extra
    // waves only help with the prologue
    const int64_t need = ceil_div(xpieces, (int64_t)kXReg * 64);
    if (p.waves < need) p.waves = (int)(need < maxw ? need : maxw);
  }
  p.SB = 1;
  if (allow_split && p.amode == AGLOBAL && p.Ng < 64 && p.tps >= 16) {
    // tiny output, long K: split K across workgroups too
    int64_t cap = 512 / p.Ng;
    if (cap < 2) cap = 2;
    int sb = (int)ceil_div(p.tps, 4);
    p.SB = (int)(sb > cap ? cap : sb);
    p.waves = maxw;
    p.tps = (int)ceil_div(p.Kt, (int64_t)p.waves * p.SB);
  }
  if (p.SB > 1) {
    p.ws_acc_bytes = M * p.Ng * p.NB * kTileN * 4;
    p.ws_bytes = p.ws_acc_bytes + (int64_t)p.Ng * 4;
  }
  return p;
}

struct GemvSeg {
  const u4* packed;
  const float* beta;
  void* y;
  int N, Nt;
  int g0;  // first output group of the segment in the grid
};

struct GemvArgs {
  const int8_t* q;  // [M][ldq] int8 (modes AGLOBAL, ALDS_Q)
  const void* x;    // [M][K] bf16/fp32 activations (mode ALDS_X)
  int x_dtype;       // BITLINEAR_BF16 or BITLINEAR_F32
  int x_vec;        // ALDS_X: rows can be read in 16-byte pieces
  int norm;         // fused modes: RMS-normalize each row before quantizing
  const float* ds;  // [M] (modes AGLOBAL, ALDS_Q)
  int M, K, Kt, tps, SB;
  int64_t ldq, ldl;
  GemvSeg seg[kGemvMaxSeg];
  const int32_t* rowsum;  // B1: per-token sum of the int8 codes
  int nseg;         // segments in use (1 for a single BitLinear)
  int glu;          // gated pair: seg[0] gate, seg[1] up, h into seg[0].y
  int y_dtype;
  int32_t* ws_acc;
  uint32_t* ws_cnt;
  // requantization of output 0 (or h) for the next BitLinear by the last
  // workgroup to finish (RQ instantiations only)
  const float* rq_src;  // fp32 rows [M][rq_k]
  int rq_k, rq_norm;
  int8_t* rq_q;         // [M][rq_ldq]
  int64_t rq_ldq;
  float* rq_ds;         // [M]
  uint32_t* rq_cnt;     // arrival counter, zero on entry and on return
};

// Tail of a requantizing launch, reached by every wave of every workgroup
// after its output stores: each wave waits for its own stores, then one
// thread releases the workgroup's outputs at agent scope and counts its
// arrival; the last workgroup to arrive acquires everyone's outputs and
// quantizes rows m < M of rq_src (optionally RMS-normalized) into
// rq_q / rq_ds, one row per wave, then resets the counter.  No workgroup
// waits for another.
__device__ void rq_tail(const GemvArgs& a) {
  __shared__ uint32_t last;
  const int wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  // The outputs were written with agent-coherent stores (written through the
  // compute die's L2); waiting for their completion makes them visible to
  // every die before the arrival is counted, without an L2 writeback.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    last = __hip_atomic_fetch_add(a.rq_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // drop stale lines of this die's caches
  }
  __syncthreads();
  if (!last) return;
  for (int m = wave; m < a.M; m += waves)
    wave_quant_row_f32(a.rq_src + (int64_t)m * a.rq_k, a.rq_k, a.rq_norm != 0, a.rq_q + (int64_t)m * a.rq_ldq,
                       a.rq_ldq, a.rq_ds + m);
  if (threadIdx.x == 0) __hip_atomic_store(a.rq_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a.seg[si] for a uniform si, field by field through selects over the fixed
// offsets of every segment
__device__ inline GemvSeg seg_select(const GemvArgs& a, int si) {
  GemvSeg s = a.seg[0];
#pragma unroll
  for (int i = 1; i < kGemvMaxSeg; ++i) {
    const bool t = si == i;
    s.packed = t ? a.seg[i].packed : s.packed;
    s.beta = t ? a.seg[i].beta : s.beta;
    s.y = t ? a.seg[i].y : s.y;
    s.N = t ? a.seg[i].N : s.N;
    s.Nt = t ? a.seg[i].Nt : s.Nt;
    s.g0 = t ? a.seg[i].g0 : s.g0;
  }
  return s;
}

__device__ inline float x_at(const void* x, int dt, int64_t i) {
  return dt == BITLINEAR_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[i])
                              : static_cast<const float*>(x)[i];
}



// Staged prologue, part 1 (issued before the weight loads, so that waiting
// for these pieces never waits for the weight stream): piece c of the
// contiguous source rows (int8 rows of act_stride bytes, or 16-byte-aligned
// bf16/fp32 rows) goes to v[r] for c = tid + r * blockDim.x.  Threads past
// the last piece load a duplicate of the last piece (never stored, and a
// duplicate cannot change a maximum).
// With more than kXReg slots, slots wholly past the last piece are skipped
// (a uniform test): short rows do not issue XR loads per thread.
template <int XR>
__device__ inline void stage_load(const u4* src, int npieces, u4 (&v)[XR]) {
  const int tid = threadIdx.x, nthr = blockDim.x;
#pragma unroll
  for (int r = 0; r < XR; ++r)
    if (XR <= kXReg || r * nthr < npieces) v[r] = src[min(tid + r * nthr, npieces - 1)];
}

// Part 2 for int8 rows: write the held pieces (and any beyond XR per
// thread) to the padded LDS rows.
template <int XR>
__device__ void stage_store_q(const GemvArgs& a, const u4 (&v)[XR], int8_t* lds) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int cpr = (int)(a.ldq / 16), npieces = a.M * cpr;
  const int rowp = (int)((a.ldl - kLdsPad) / 16);  // pieces of a row the kernel reads
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int c = tid + r * nthr;
    if (c < npieces) {
      const int m = c / cpr, pc = c - m * cpr;
      if (pc < rowp) *reinterpret_cast<u4*>(lds + (int64_t)m * a.ldl + pc * 16) = v[r];
    }
  }
  __syncthreads();
}

// The same copy for rows the threads cannot hold in registers; issued before
// the weight loads (a loop of loads after them would make every later wait
// cover the weight stream).
__device__ void copy_rows_q(const GemvArgs& a, int8_t* lds) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int cpr = (int)(a.ldq / 16), npieces = a.M * cpr;
  const int rowp = (int)((a.ldl - kLdsPad) / 16);
  const u4* src = reinterpret_cast<const u4*>(a.q);
  for (int c = tid; c < npieces; c += nthr) {
    const int m = c / cpr, pc = c - m * cpr;
    if (pc < rowp) *reinterpret_cast<u4*>(lds + (int64_t)m * a.ldl + pc * 16) = src[c];
  }
  __syncthreads();
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// max |x| over a 16-byte piece (8 bf16 or 4 fp32 values) as fp32 bits: with
// the sign bits cleared the bit patterns order like the magnitudes, so the
// maximum is taken on integers (packed 16-bit for bf16).
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

// One int8 code q = rint(x * qs) as a byte.  |x * qs| <= 127 * (1 + 2^-23)
// because |x| <= g and qs = fl(127 / g), so adding 1.5 * 2^23 rounds the
// product to the nearest integer, ties to even (the sum lies in [2^23, 2^24)
// where the float spacing is 1), the integer sits in the low mantissa bits,
// and the clamp to [-127, 127] can never act.  Multiply and add are separate
// roundings (no contraction), exactly as rint(fl(x * qs)).
__device__ inline uint32_t qbyte(float x, float qs) {
  return __float_as_uint(__fadd_rn(__fmul_rn(x, qs), 12582912.0f)) & 0xffu;
}
// The same word before the mask (the code is its low byte), and the low
// bytes of four such words packed in order by byte permutes (v_perm_b32
// picks bytes of {S0, S1}, S1 bytes 0..3, S0 bytes 4..7, selector 12 = zero):
// three operations per four codes instead of masks and shifts.
__device__ inline uint32_t qword(float x, float qs) {
  return __float_as_uint(__fadd_rn(__fmul_rn(x, qs), 12582912.0f));
}
__device__ inline uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a0, b0, 0, 0
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);  // c0, d0, 0, 0
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);              // a0, b0, c0, d0
}

// Quantize one 16-byte piece (8 bf16 or 4 fp32 values) into LDS at dst.
__device__ inline void piece_quant_store(const u4 v, bool bf16, float qs, int8_t* dst) {
  if (bf16) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = pack_low_bytes(qword(__uint_as_float(v[2 * h] << 16), qs), qword(__uint_as_float(v[2 * h] & 0xffff0000u), qs),
                            qword(__uint_as_float(v[2 * h + 1] << 16), qs),
                            qword(__uint_as_float(v[2 * h + 1] & 0xffff0000u), qs));
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = pack_low_bytes(qword(__uint_as_float(v[0]), qs), qword(__uint_as_float(v[1]), qs),
                                                       qword(__uint_as_float(v[2]), qs), qword(__uint_as_float(v[3]), qs));
  }
}

// Sum of squares of a piece's values in fp64 (each square exact).
__device__ inline double piece_sumsq(const u4 v, bool bf16) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (bf16) {
      const double lo = __uint_as_float(v[j] << 16), hi = __uint_as_float(v[j] & 0xffff0000u);
      s += lo * lo;
      s += hi * hi;
    } else {
      const double e = __uint_as_float(v[j]);
      s += e * e;
    }
  }
  return s;
}

// RMS normalization scale r = 1 / sqrt((float)(S / K) + 1e-5) (fp32, correctly
// rounded division and root), as the standalone quantizer applies it.
__device__ inline float rms_scale(double sumsq, int K) {
  const float ms = (float)(sumsq / (double)K);
  return 1.0f / sqrtf(ms + 1e-5f);
}

// Quantize a piece after scaling its values by r (bf16 widens exactly to fp32).
__device__ inline void piece_quant_store_norm(const u4 v, bool bf16, float r, float qs, int8_t* dst) {
  auto sc = [&](uint32_t bits) { return __float_as_uint(__fmul_rn(__uint_as_float(bits), r)); };
  if (bf16) {
    piece_quant_store(u4{sc(v[0] << 16), sc(v[0] & 0xffff0000u), sc(v[1] << 16), sc(v[1] & 0xffff0000u)}, false, qs, dst);
    piece_quant_store(u4{sc(v[2] << 16), sc(v[2] & 0xffff0000u), sc(v[3] << 16), sc(v[3] & 0xffff0000u)}, false, qs,
                      dst + 4);
  } else {
    piece_quant_store(u4{sc(v[0]), sc(v[1]), sc(v[2]), sc(v[3])}, false, qs, dst);
  }
}

// Row of piece c (cpr pieces per row); exact for c < 2^24 (the float error of
// (c + 0.5) / cpr is far below the 0.5 / cpr margin to a row boundary).
__device__ inline int piece_row(int c, int M, float inv_cpr) {
  return M == 1 ? 0 : (int)(((float)c + 0.5f) * inv_cpr);
}

// Part 2 for bf16/fp32 rows (16-byte aligned, K a multiple of the piece) that
// the threads hold entirely in registers (M * K / piece <= kXReg * threads):
// gamma_m = max |x[m][:]| from the held pieces (per-wave maxima in LDS slots,
// combined by thread m), then each piece quantized with
// q = rint(x * (127 / max(gamma, 1e-5))) into LDS.  `slots` holds at least
// waves * M words, `sq` waves * M doubles.  With a.norm the row is first
// RMS-normalized (per-wave fp64 sums of squares in `sq`, added in wave order):
// the quantizer sees fl(x * r), whose maximum is fl(gamma * r).
template <bool NORM>
__device__ void stage_store_x(const GemvArgs& a, const u4 (&v)[kXReg], int8_t* lds, uint32_t* slots, double* sq,
                              float* row_g, float* row_qs, float* row_r) {
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6, waves = nthr >> 6;
  const bool bf16 = a.x_dtype == BITLINEAR_BF16;
  const int per16 = bf16 ? 8 : 4;
  const int M = a.M, cpr = a.K / per16, npieces = M * cpr;
  const float inv_cpr = 1.0f / (float)cpr;
  const int64_t Kp = (int64_t)a.Kt * kTileK;
  // zero the padding columns [K, Kp) of every row (4-byte stores)
  const int padw = (int)((Kp - a.K) / 4);
  for (int i = tid; i < M * padw; i += nthr) {
    const int m = i / padw;
    *reinterpret_cast<uint32_t*>(lds + (int64_t)m * a.ldl + a.K + 4 * (i - m * padw)) = 0u;
  }
  constexpr bool norm = NORM;
  // row of each held piece (-1 past the last piece), and its maximum
  int prow[kXReg];
  uint32_t pmax[kXReg];
#pragma unroll
  for (int r = 0; r < kXReg; ++r) {
    const int c = tid + r * nthr;
    prow[r] = c < npieces ? piece_row(c, M, inv_cpr) : -1;
    pmax[r] = piece_absmax_bits(v[r], bf16);
  }
  for (int m = 0; m < M; ++m) {
    uint32_t amax = 0;
    double s2 = 0.0;
#pragma unroll
    for (int r = 0; r < kXReg; ++r) {
      if (prow[r] == m) {
        amax = max(amax, pmax[r]);
        if (norm) s2 += piece_sumsq(v[r], bf16);
      }
    }
    amax = wave_max_u32(amax);
    if (lane == 0) slots[wave * M + m] = amax;
    if (norm) {
      s2 = wave_sum_f64(s2);
      if (lane == 0) sq[wave * M + m] = s2;
    }
  }
  __syncthreads();
  if (tid < M) {
    uint32_t g = 0;
    for (int w = 0; w < waves; ++w) g = max(g, slots[w * M + tid]);
    float gamma = __uint_as_float(g);
    if (norm) {
      double s2 = 0.0;
      for (int w = 0; w < waves; ++w) s2 += sq[w * M + tid];
      const float rn = rms_scale(s2, a.K);
      row_r[tid] = rn;
      gamma = __fmul_rn(gamma, rn);
    }
    const float gm = fmaxf(gamma, 1e-5f);
    row_g[tid] = gm;
    row_qs[tid] = 127.0f / gm;  // IEEE division, as the standalone quantizer
  }
  __syncthreads();
  auto quant = [&](const u4 p, int c, int m) {
    int8_t* dst = lds + (int64_t)m * a.ldl + (c - m * cpr) * per16;
    if (norm)
      piece_quant_store_norm(p, bf16, row_r[m], row_qs[m], dst);
    else
      piece_quant_store(p, bf16, row_qs[m], dst);
  };
#pragma unroll
  for (int r = 0; r < kXReg; ++r)
    if (prow[r] >= 0) quant(v[r], tid + r * nthr, prow[r]);
  __syncthreads();
}

// The same for one token row, with less bookkeeping: the slots a wave holds
// are skipped by a uniform branch past the last piece, every thread combines
// the per-wave maxima (and sums of squares) itself, in wave order, so one
// barrier fewer is needed.
template <bool NORM>
__device__ void stage_store_x1(const GemvArgs& a, const u4 (&v)[kXReg], int8_t* lds, uint32_t* slots, double* sq,
                               float* row_g, float* row_r) {
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6, waves = nthr >> 6;
  const bool bf16 = a.x_dtype == BITLINEAR_BF16;
  const int per16 = bf16 ? 8 : 4;
  const int npieces = a.K / per16;
  const int nslots = (npieces + nthr - 1) / nthr;  // uniform
  const int64_t Kp = (int64_t)a.Kt * kTileK;
  for (int64_t k = a.K + 4 * (int64_t)tid; k < Kp; k += 4 * nthr) *reinterpret_cast<uint32_t*>(lds + k) = 0u;
  uint32_t amax = 0;
  double s2 = 0.0;
#pragma unroll
  for (int r = 0; r < kXReg; ++r) {
    if (r < nslots && tid + r * nthr < npieces) {
      amax = max(amax, piece_absmax_bits(v[r], bf16));
      if (NORM) s2 += piece_sumsq(v[r], bf16);
    }
  }
  amax = wave_max_u32(amax);
  if (NORM) {
    s2 = wave_sum_f64(s2);
  }
  if (lane == 0) {
    slots[wave] = amax;
    if (NORM) sq[wave] = s2;
  }
  __syncthreads();
  uint32_t g = 0;
  for (int w = 0; w < waves; ++w) g = max(g, slots[w]);
  float gamma = __uint_as_float(g), rn = 1.0f;
  if (NORM) {
    double t = 0.0;
    for (int w = 0; w < waves; ++w) t += sq[w];
    rn = rms_scale(t, a.K);
    gamma = __fmul_rn(gamma, rn);
  }
  const float gm = fmaxf(gamma, kEpsX);
  const float qs = 127.0f / gm;  // IEEE division, as the standalone quantizer
  if (tid == 0) {
    row_g[0] = gm;
    if (NORM) row_r[0] = rn;
  }
#pragma unroll
  for (int r = 0; r < kXReg; ++r) {
    const int c = tid + r * nthr;
    if (r < nslots && c < npieces) {
      if (NORM)
        piece_quant_store_norm(v[r], bf16, rn, qs, lds + c * per16);
      else
        piece_quant_store(v[r], bf16, qs, lds + c * per16);
    }
  }
  __syncthreads();
}

// ALDS_XS prologue, for rows that are not whole 16-byte pieces (unaligned x
// or K not a multiple of the piece): row_g[m] = max(max_k |x[m][k]|, 1e-5)
// (of the normalized row with a.norm, as stage_store_x), then the int8 rows
// into LDS, element by element.
template <bool NORM>
__device__ void quantize_rows_scalar(const GemvArgs& a, int8_t* lds, double* sq, float* row_g, float* row_qs,
                                     float* row_r) {
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6, waves = nthr >> 6;
  const int M = a.M;
  constexpr bool norm = NORM;
  const int64_t Kp = (int64_t)a.Kt * kTileK;
  if (tid < 64) row_g[tid] = 0.0f;
  __syncthreads();
  for (int m = 0; m < M; ++m) {
    float amax = 0.0f;
    double s2 = 0.0;
    for (int k = tid; k < a.K; k += nthr) {
      const float xv = x_at(a.x, a.x_dtype, (int64_t)m * a.K + k);
      amax = fmaxf(amax, fabsf(xv));
      if (norm) s2 += (double)xv * (double)xv;
    }
    amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));  // amax >= 0: bits order like values
    // |x| >= 0, so the fp32 bit patterns order like the values
    if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(&row_g[m]), __float_as_uint(amax));
    if (norm) {
      s2 = wave_sum_f64(s2);
      if (lane == 0) sq[wave * M + m] = s2;
    }
  }
  __syncthreads();
  if (tid < M) {
    float gamma = row_g[tid];
    if (norm) {
      double s2 = 0.0;
      for (int w = 0; w < waves; ++w) s2 += sq[w * M + tid];
      const float rn = rms_scale(s2, a.K);
      row_r[tid] = rn;
      gamma = __fmul_rn(gamma, rn);
    }
    const float gm = fmaxf(gamma, kEpsX);
    row_g[tid] = gm;
    row_qs[tid] = 127.0f / gm;  // IEEE division, as the standalone quantizer
  }
  __syncthreads();
  for (int m = 0; m < M; ++m) {
    const float qs = row_qs[m], rn = norm ? row_r[m] : 1.0f;
    int8_t* lrow = lds + (int64_t)m * a.ldl;
    for (int k = 4 * tid; k < Kp; k += 4 * nthr) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k + j < a.K) {
          const float xv = x_at(a.x, a.x_dtype, (int64_t)m * a.K + k + j);
          w |= qbyte(norm ? __fmul_rn(xv, rn) : xv, qs) << (8 * j);
        }
      *reinterpret_cast<uint32_t*>(lrow + k) = w;
    }
  }
  __syncthreads();
}

// Expand step s (0..7) of a B1 lane chunk: bits 16 (s % 2) .. +15 of dword
// s / 2 become 16 bytes in {0, 1} (bit j -> byte j).  A nibble times
// 0x00204081 places its bits 0..3 at bits 0, 8, 16, 24 without carries.
__device__ inline v4i b1_field(const u4 w, int s) {
  const uint32_t bits = w[s >> 1] >> (16 * (s & 1));
  v4i r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = (int)((((bits >> (4 * q)) & 0xFu) * 0x00204081u) & 0x01010101u);
  return r;
}

// Base-3 digits of the four bytes of dw, as bytes: d[s] byte j = digit s of
// byte j.  Bytes 0/2 and 1/3 are processed as 16-bit pairs; q_s = floor(b /
// 3^s) = (b * m_s) >> sh_s is exact for b <= 242 with products below 2^16.
typedef unsigned short us2v __attribute__((ext_vector_type(2)));
__device__ inline void b3_digits(uint32_t dw, uint32_t (&d)[5]) {
  const us2v e = __builtin_bit_cast(us2v, dw & 0x00FF00FFu);
  const us2v o = __builtin_bit_cast(us2v, (dw >> 8) & 0x00FF00FFu);
  auto qd = [](us2v x, unsigned short m, unsigned short sh) -> us2v {
    return (us2v)((x * (us2v){m, m}) >> (us2v){sh, sh});
  };
  const us2v three = {3, 3};
  const us2v e1 = qd(e, 171, 9), e2 = qd(e, 228, 11), e3 = qd(e, 152, 12), e4 = qd(e, 203, 14);
  const us2v o1 = qd(o, 171, 9), o2 = qd(o, 228, 11), o3 = qd(o, 152, 12), o4 = qd(o, 203, 14);
  const us2v de[5] = {e - three * e1, e1 - three * e2, e2 - three * e3, e3 - three * e4, e4};
  const us2v dd[5] = {o - three * o1, o1 - three * o2, o2 - three * o3, o3 - three * o4, o4};
#pragma unroll
  for (int s = 0; s < 5; ++s) d[s] = __builtin_bit_cast(uint32_t, de[s]) | (__builtin_bit_cast(uint32_t, dd[s]) << 8);
}

// Byte offset within a token row of the 16 activation bytes that lanes
// 16 g4 .. 16 g4 + 15 use in MFMA step i of k-tile kt (KT columns per tile).
// Rows read from global memory are act_stride(K) bytes, which can be shorter
// than the k-tiles of a base-3 matrix (320 columns): those reads are clamped
// to the row's last 16 bytes.  Every column they stand for is past K (the row
// length and the offsets are multiples of 16), where the weight codes are 0
// (base 3: c = 0), so the bytes read there add nothing, and the rowsum
// correction covers the real columns only.
__host__ __device__ inline int64_t act_col(int kt, int i, int g4, int KT, int64_t row_bytes, bool clamp) {
  const int64_t c = (int64_t)kt * KT + 64 * i + 16 * g4;
  return clamp && c > row_bytes - 16 ? row_bytes - 16 : c;
}

template <int MB, int NB, int AM, bool NORM, int FMT = 0, int kU = ring_depth(MB, NB, AM, FMT), bool RQ = false,
          bool BIGX = false>
__global__ __launch_bounds__(64 * max_waves(MB, NB)) void gemv_t2_kernel(const GemvArgs a) {
  constexpr int KT = tile_cols(FMT), NS = KT / 64;  // columns and MFMA steps per k-tile
  // wide plans (one token block, 4 or more output blocks): interleaved k-tiles
  constexpr bool KINT = MB == 1 && NB >= 4 && FMT == 0 && AM != AGLOBAL;
  constexpr int E = MB * NB * 4;  // accumulator values per lane
  constexpr int UA = AM == AGLOBAL ? kU : 1;
  __shared__ int red[E][64];
  constexpr bool FUSED = AM == ALDS_X || AM == ALDS_XS;
  __shared__ float row_g[FUSED ? 64 : 1];   // fused: per-row g = max(max |x|, 1e-5)
  __shared__ float row_qs[FUSED ? 64 : 1];  // fused: per-row 127 / max(gamma, eps)
  __shared__ float row_r[NORM ? 64 : 1];   // fused with normalization: per-row RMS scale
  __shared__ double sq_slots[NORM ? max_waves(MB) * 16 * MB : 1];  // per-wave, per-row sums of squares
  extern __shared__ __attribute__((aligned(16))) int8_t act_lds[];  // [M][ldl]

  if constexpr (kLdsPoison) {  // LDS self-test builds
    lds_poison(&red[0][0], (int)sizeof(red));
    lds_poison(row_g, (int)sizeof(row_g));
    lds_poison(row_qs, (int)sizeof(row_qs));
    lds_poison(row_r, (int)sizeof(row_r));
    lds_poison(sq_slots, (int)sizeof(sq_slots));
    if (AM != AGLOBAL) lds_poison(act_lds, (int)(a.M * a.ldl));
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, waves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int grp = blockIdx.x / a.SB, sb = blockIdx.x - grp * a.SB;
  const int split = sb * waves + wave;
  const int k0 = split * a.tps;
  const int k1 = min(k0 + a.tps, a.Kt);
  // wide plans: k-tiles wave, wave + waves, ... (ns of them)
  const int ns = KINT ? (a.Kt > wave ? (a.Kt - wave + waves - 1) / waves : 0) : 0;
  auto kof = [&](int s) { return wave + s * waves; };
  // Segment of this workgroup (uniform).  The segment fields come from fixed
  // argument offsets and a select on the index, so no argument load waits
  // for the index (each such wait is one more round trip before the first
  // weight load).
  int si = 0;
#pragma unroll
  for (int i = 1; i < kGemvMaxSeg; ++i) si = i < a.nseg && grp >= a.seg[i].g0 ? i : si;
  const GemvSeg sg = seg_select(a, si);
  const int lg = grp - sg.g0;                // output group within the segment
  const int nb0 = a.glu ? lg : lg * NB;      // first 16-row output block
  const int r16 = lane & 15, g4 = lane >> 4;
  const int M = a.M;

  v4i acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = v4i{0, 0, 0, 0};

  const u4* bptr[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    // blocks past Nt are masked at the store; a gated pair reads block nb0
    // of the gate (j = 0) and of the up matrix (j = 1)
    const int nb = min(a.glu ? nb0 : nb0 + j, sg.Nt - 1);
    bptr[j] = (a.glu ? a.seg[j].packed : sg.packed) + (int64_t)nb * a.Kt * 64 + lane;
  }
  // Activation operand rows.  Lanes of token rows >= M read row M-1 instead:
  // their accumulators are never stored, so the loads need no branch.
  int64_t aoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) aoff[mb] = (int64_t)min(mb * 16 + r16, M - 1) * (AM == AGLOBAL ? a.ldq : a.ldl);

  u4 wbuf[kU][NB];
  v4i abuf[UA][MB][NS];
  auto load_w = [&](int slot, int kt) {
#pragma unroll
    for (int j = 0; j < NB; ++j) wbuf[slot][j] = __builtin_nontemporal_load(bptr[j] + (int64_t)kt * 64);
  };
  auto load_a = [&](int slot, int kt) {
    const int8_t* base = AM == AGLOBAL ? a.q : act_lds;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < NS; ++i)
        abuf[slot][mb][i] = *reinterpret_cast<const v4i*>(
            base + aoff[mb] + act_col(kt, i, g4, KT, a.ldq, AM == AGLOBAL && FMT == 2));
  };
  auto mma_tile = [&](int slot, int kt) {
    const int as = AM == AGLOBAL ? slot : 0;
    if (AM != AGLOBAL) load_a(0, kt);  // LDS operands: read at use
    v4i b3ops[FMT == 2 ? NB : 1][FMT == 2 ? 5 : 1];
    if constexpr (FMT == 2) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        uint32_t dg[4][5];
#pragma unroll
        for (int w = 0; w < 4; ++w) b3_digits(wbuf[slot][j][w], dg[w]);
#pragma unroll
        for (int st = 0; st < 5; ++st) b3ops[j][st] = v4i{(int)dg[0][st], (int)dg[1][st], (int)dg[2][st], (int)dg[3][st]};
      }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const v4i b = FMT == 2 ? b3ops[FMT == 2 ? j : 0][FMT == 2 ? i : 0]
                               : (FMT == 1 ? b1_field(wbuf[slot][j], i) : t2_field(wbuf[slot][j], i));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][j] = mfma16(abuf[as][mb][i], b, acc[mb][j]);
      }
  };

  const bool has_work = KINT ? ns > 0 : k0 < k1;
  // activation pieces first (few, cache-resident), then the weight stream.
  // Rows the threads cannot hold in registers (and rows that are not whole
  // pieces) are quantized completely before the weight loads are issued: a
  // loop of activation loads after them would make every later wait cover
  // the whole weight stream.
  // wide plans with long int8 rows (BIGX) hold twice the pieces: those rows
  // may use most of the unit's LDS, and 8 waves leave the registers for it
  constexpr int XR = BIGX ? 2 * kXReg : kXReg;
  u4 stage[XR];
  const int xpieces = a.M * (a.K / (a.x_dtype == BITLINEAR_BF16 ? 8 : 4));
  const bool held = xpieces <= kXReg * (int)blockDim.x;
  if constexpr (AM == ALDS_X) {
    if (held)
      stage_load(static_cast<const u4*>(a.x), xpieces, stage);
    else
      quantize_rows_scalar<NORM>(a, act_lds, sq_slots, row_g, row_qs, row_r);
  }
  if constexpr (AM == ALDS_XS) quantize_rows_scalar<NORM>(a, act_lds, sq_slots, row_g, row_qs, row_r);
  if constexpr (AM == ALDS_Q) {
    if (a.M * (int)(a.ldq / 16) <= XR * (int)blockDim.x)
      stage_load(reinterpret_cast<const u4*>(a.q), a.M * (int)(a.ldq / 16), stage);
    else
      copy_rows_q(a, act_lds);
  }
  // Unconditional, so the wait for the staged pieces never has to assume a
  // path without weight loads (a wave without k-tiles reads tile 0 of its
  // first block, in bounds, and never uses it).
  if constexpr (KINT) {
#pragma unroll
    for (int u = 0; u < kU; ++u) load_w(u, has_work ? kof(min(u, ns - 1)) : 0);
  } else {
    const int kfirst = has_work ? k0 : 0, klast = has_work ? k1 - 1 : 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) load_w(u, min(kfirst + u, klast));
  }
  // keep the compiler from hoisting work on the staged pieces above the
  // weight loads (that would wait for the pieces before the stream starts)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (AM == ALDS_Q) {
    if (a.M * (int)(a.ldq / 16) <= XR * (int)blockDim.x) stage_store_q(a, stage, act_lds);
  }
  if constexpr (AM == ALDS_X) {
    if (held) {
      if (M == 1)
        stage_store_x1<NORM>(a, stage, act_lds, reinterpret_cast<uint32_t*>(&red[0][0]), sq_slots, row_g, row_r);
      else
        stage_store_x<NORM>(a, stage, act_lds, reinterpret_cast<uint32_t*>(&red[0][0]), sq_slots, row_g, row_qs,
                            row_r);
    }
  }

  if (KINT && has_work) {
    // ring of kU k-steps of NB tiles; each tile is re-loaded right after its
    // last use, and only while k-steps remain (no re-loads past the end)
    auto step = [&](int slot, int kt, int ktn, auto reload) {
      load_a(0, kt);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < NS; ++i) acc[0][j] = mfma16(abuf[0][0][i], t2_field(wbuf[slot][j], i), acc[0][j]);
        if constexpr (decltype(reload)::value) {
          wbuf[slot][j] = __builtin_nontemporal_load(bptr[j] + (int64_t)ktn * 64);
          // keep the re-load here: scheduled after the whole step, the wave
          // would wait for every tile in flight before issuing the next ones
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    int s = 0;
    for (; s + 2 * kU <= ns; s += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) step(u, kof(s + u), kof(s + u + kU), std::true_type{});
    }
    const int rem = ns - s;  // k-steps left, in [kU, 2 kU) once ns >= kU
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u + kU < rem)
        step(u, kof(s + u), kof(s + u + kU), std::true_type{});
      else if (u < rem)
        step(u, kof(s + u), 0, std::false_type{});
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (u + kU < rem) step(u, kof(s + kU + u), 0, std::false_type{});
  } else if (has_work) {
    // ring of kU k-tiles in flight; re-loads past the end read tile k1-1
    // again (in bounds) and are never used
    if constexpr (AM == AGLOBAL) {
#pragma unroll
      for (int u = 0; u < kU; ++u) load_a(u, min(k0 + u, k1 - 1));
    }
    int kt = k0;
    for (; kt + kU <= k1; kt += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        mma_tile(u, kt + u);
        load_w(u, min(kt + u + kU, k1 - 1));
        if constexpr (AM == AGLOBAL) load_a(u, min(kt + u + kU, k1 - 1));
      }
    }
    const int rem = k1 - kt;
#pragma unroll
    for (int u = 0; u < kU - 1; ++u)
      if (u < rem) mma_tile(u, kt + u);
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
        for (int r = 0; r < 4; ++r)  // rows mb * 16 + 4 g4 + r: none below M once mb * 16 + r >= M
          if (mb * 16 + r < M) atomicAdd(&red[(mb * NB + j) * 4 + r][lane], acc[mb][j][r]);
    __syncthreads();
    if (wave != 0) {
      if constexpr (RQ) rq_tail(a);
      return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mb][j][r] = red[(mb * NB + j) * 4 + r][lane];
  }

  // ---- combine workgroups (K split across the grid; AGLOBAL plans only)
  if (AM == AGLOBAL && a.SB > 1) {
    const int ldw = gridDim.x / a.SB * NB * kTileN;  // workspace row length
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mb * 16 + 4 * g4 + r;
          const int n = (nb0 + j) * kTileN + r16;
          if (m < M)
            __hip_atomic_fetch_add(a.ws_acc + (int64_t)m * ldw + n, acc[mb][j][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    __threadfence();
    int last = 0;
    if (lane == 0)
      last = __hip_atomic_fetch_add(a.ws_cnt + grp, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(a.SB - 1);
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
          acc[mb][j][r] = m < M ? __hip_atomic_exchange(a.ws_acc + (int64_t)m * ldw + n, 0, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                : 0;
        }
    if (lane == 0) __hip_atomic_store(a.ws_cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- dequantize and store: lane holds rows 4*g4 + r of each token block,
  //      column r16 of each output block
  if (a.glu) {
    // h = (r * r) * y_up with r = max(y_gate, +0), each y dequantized as below
    const float bg = *a.seg[0].beta, bu = *a.seg[1].beta;
    const int n = nb0 * kTileN + r16;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mb * 16 + 4 * g4 + r;
        if (m >= M || n >= sg.N) continue;
        const float dsm = FUSED ? row_g[m] / 127.0f : a.ds[m];
        const float yg = (float)(acc[mb][0][r] >> 6) * (dsm * bg);
        const float yu = (float)(acc[mb][NB - 1][r] >> 6) * (dsm * bu);
        const float rg = yg > 0.0f ? yg : 0.0f;
        float* dst = static_cast<float*>(sg.y) + (int64_t)m * sg.N + n;
        if constexpr (RQ)
          __hip_atomic_store(dst, __fmul_rn(__fmul_rn(rg, rg), yu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *dst = __fmul_rn(__fmul_rn(rg, rg), yu);
      }
    if constexpr (RQ) rq_tail(a);
    return;
  }
  const float bt = *sg.beta;
  if constexpr (FUSED && NB < 4) {
    // one or two output blocks: the row scales are in LDS and a type switch
    // per element stays a short run of code (measured no slower here than
    // the single dispatch below; 6912 -> 2560 at one token 4.65 against 4.8
    // us)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mb * 16 + 4 * g4 + r;
        if (m >= M) continue;
        const float scale = (row_g[m] / 127.0f) * bt;  // g of the normalized row with a.norm
        const int rs = FMT ? a.rowsum[m] : 0;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int n = (nb0 + j) * kTileN + r16;
          const int v = FMT == 1 ? (2 * acc[mb][j][r] - rs) * 64
                                 : (FMT == 2 ? (acc[mb][j][r] - rs) * 64 : acc[mb][j][r]);
          if (n < sg.N) store_out(sg.y, a.y_dtype, (int64_t)m * sg.N + n, v, scale);
        }
      }
  } else {
    // Every row scale is read before the first store (a global load between
    // stores would wait for all of them: vmcnt retires in order; fused
    // launches hold them in LDS), and the output type is dispatched once,
    // outside the store loops: with many output blocks (the wide plans) a
    // type switch per element spreads the epilogue over far-apart code
    // blocks, and every workgroup reaches it with those instruction lines
    // not yet cached (on 8192 -> 28672 at one token that alone held each
    // workgroup ~0.4 us after its reduction).
    float scale[MB][4];
    int rsv[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mb * 16 + 4 * g4 + r;
        scale[mb][r] = 0.0f, rsv[mb][r] = 0;
        if (m < M) {
          // fused: g of the (normalized) row from the prologue, ds = g / 127
          scale[mb][r] = (FUSED ? row_g[m] / 127.0f : a.ds[m]) * bt;
          rsv[mb][r] = FMT ? a.rowsum[m] : 0;
        }
      }
    auto emit = [&](auto ytype) {
      constexpr int YD = decltype(ytype)::value;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mb * 16 + 4 * g4 + r;
          if (m >= M) continue;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int n = (nb0 + j) * kTileN + r16;
            // B1: sum q * (2 b - 1) = 2 sum q * b - rowsum; B3: sum q * (c - 1) =
            // sum q * c - rowsum; both scaled as the T2 sums (64 t)
            const int v = FMT == 1 ? (2 * acc[mb][j][r] - rsv[mb][r]) * 64
                                   : (FMT == 2 ? (acc[mb][j][r] - rsv[mb][r]) * 64 : acc[mb][j][r]);
            if (n < sg.N) {
              if constexpr (RQ && (YD == BITLINEAR_F32 || YD == BITLINEAR_F32_ADD)) {
                // agent-coherent store: the last workgroup requantizes these rows
                float* dst = static_cast<float*>(sg.y) + (int64_t)m * sg.N + n;
                float val = (float)(v >> 6) * scale[mb][r];
                if constexpr (YD == BITLINEAR_F32_ADD) val = __fadd_rn(*dst, val);
                __hip_atomic_store(dst, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              } else {
                store_out_t<YD>(sg.y, (int64_t)m * sg.N + n, v, scale[mb][r]);
              }
            }
          }
        }
    };
    switch (a.y_dtype) {
      case BITLINEAR_I32: emit(std::integral_constant<int, BITLINEAR_I32>{}); break;
      case BITLINEAR_F32: emit(std::integral_constant<int, BITLINEAR_F32>{}); break;
      case BITLINEAR_F32_ADD: emit(std::integral_constant<int, BITLINEAR_F32_ADD>{}); break;
      default: emit(std::integral_constant<int, BITLINEAR_BF16>{}); break;
    }
  }
  if constexpr (RQ) rq_tail(a);
}

template <int MB, int NB, int AM, bool NORM, int FMT = 0, bool RQ = false, bool BIGX = false>
hipError_t launch_t(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  constexpr int KU = ring_depth(MB, NB, AM, FMT);
  if constexpr (AM != AGLOBAL) {
    // static LDS plus the largest activation rows can pass the default 64 KB
    // per workgroup: raise the limit (once per device)
    static LdsLimit lim;
    constexpr bool wide = MB == 1 && NB >= 4 && FMT == 0;
    const hipError_t attr =
        ensure_lds_limit(lim, reinterpret_cast<const void*>(&gemv_t2_kernel<MB, NB, AM, NORM, FMT, KU, RQ, BIGX>),
                         (int)(wide ? kWideLdsBytes : kDecodeLdsBytes));
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((gemv_t2_kernel<MB, NB, AM, NORM, FMT, KU, RQ, BIGX>), dim3((unsigned)(p.Ng * p.SB)),
                     dim3(64 * p.waves), (size_t)p.lds_bytes, s, a);
  return hipGetLastError();
}

template <int AM, bool NORM = false, int FMT = 0, bool RQ = false>
hipError_t dispatch_mb_nb(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
#define BL_GEMV_CASE(mb, nb) \
  if (p.MB == mb && p.NB == nb) return launch_t<mb, nb, AM, NORM, FMT, RQ>(p, a, s)
  // the (MB, NB) pairs make_plan can produce for this mode
  BL_GEMV_CASE(1, 1);
  BL_GEMV_CASE(1, 2);
  BL_GEMV_CASE(2, 1);
  BL_GEMV_CASE(2, 2);
  BL_GEMV_CASE(3, 1);
  BL_GEMV_CASE(4, 1);
  BL_GEMV_CASE(3, 2);  // AGLOBAL, and gated pairs in every mode
  BL_GEMV_CASE(4, 2);
  if constexpr (AM == AGLOBAL && FMT == 0 && !RQ) BL_GEMV_CASE(2, 4);
  if constexpr (AM == ALDS_Q && FMT == 0 && !RQ) {  // wide plans with long int8 rows
    if (p.bigx) {
      if (p.NB == 4) return launch_t<1, 4, AM, NORM, FMT, RQ, true>(p, a, s);
      if (p.NB == 5) return launch_t<1, 5, AM, NORM, FMT, RQ, true>(p, a, s);
      if (p.NB == 6) return launch_t<1, 6, AM, NORM, FMT, RQ, true>(p, a, s);
      if (p.NB == 7) return launch_t<1, 7, AM, NORM, FMT, RQ, true>(p, a, s);
      if (p.NB == 8) return launch_t<1, 8, AM, NORM, FMT, RQ, true>(p, a, s);
      return hipErrorInvalidValue;
    }
  }
  if constexpr (AM != AGLOBAL && FMT == 0 && !RQ) {  // wide plans
    BL_GEMV_CASE(1, 4);
    BL_GEMV_CASE(1, 5);
    BL_GEMV_CASE(1, 6);
    BL_GEMV_CASE(1, 7);
    BL_GEMV_CASE(1, 8);
  }
#undef BL_GEMV_CASE
  return hipErrorInvalidValue;
}

hipError_t dispatch(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  switch (p.amode) {
    case ALDS_Q: return dispatch_mb_nb<ALDS_Q>(p, a, s);
    case ALDS_X:
      if (a.norm) return a.x_vec ? dispatch_mb_nb<ALDS_X, true>(p, a, s) : dispatch_mb_nb<ALDS_XS, true>(p, a, s);
      return a.x_vec ? dispatch_mb_nb<ALDS_X>(p, a, s) : dispatch_mb_nb<ALDS_XS>(p, a, s);
    default: return dispatch_mb_nb<AGLOBAL>(p, a, s);
  }
}

GemvArgs make_args(const GemvPlan& p, int64_t M, int64_t K, int64_t N, const uint8_t* packed, const float* beta,
                   void* y, int y_dtype, void* ws, int fmt = 0) {
  GemvArgs a{};
  a.M = (int)M;
  a.K = (int)K;
  a.Kt = p.Kt;
  a.tps = p.tps;
  a.SB = p.SB;
  a.ldq = (int64_t)p.Kt * tile_cols(fmt);
  a.ldl = lds_row(K, fmt);
  a.nseg = 1;
  a.seg[0] = GemvSeg{reinterpret_cast<const u4*>(packed), beta, y, (int)N, p.Nt, 0};
  a.y_dtype = y_dtype;
  if (p.SB > 1) {
    a.ws_acc = static_cast<int32_t*>(ws);
    a.ws_cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + p.ws_acc_bytes);
  }
  return a;
}

// Plan and arguments for several segments (glu: exactly two of one shape).
// The plan is the single-matrix plan for the summed output rows (one per
// matrix for a gated pair), without any K split across workgroups.
bool make_multi(int64_t M, int64_t K, int count, const uint8_t* const* packed, const float* const* beta,
                const int64_t* N, void* const* y, int y_dtype, bool glu, bool fuse, int64_t xpieces, GemvPlan& p,
                GemvArgs& a) {
  if (count < 1 || count > kGemvMaxSeg || (glu && (count != 2 || N[0] != N[1]))) return false;
  int64_t ntot = 0;
  for (int i = 0; i < count; ++i) ntot += N[i];
  p = make_plan(M, glu ? N[0] : ntot, K, fuse, false, xpieces);
  if (glu) p.NB = 2;
  a = make_args(p, M, K, N[0], packed[0], beta[0], y[0], y_dtype, nullptr);
  a.nseg = count;
  a.glu = glu;
  int g = 0;
  for (int i = 0; i < count; ++i) {
    const int Nt = (int)ceil_div(N[i], kTileN);
    a.seg[i] = GemvSeg{reinterpret_cast<const u4*>(packed[i]), beta[i], y[i], (int)N[i], Nt, g};
    if (!glu) g += (int)ceil_div(Nt, p.NB);
  }
  p.Ng = glu ? a.seg[0].Nt : g;
  return true;
}

void set_x(GemvArgs& a, const void* x, int x_dtype, int64_t K) {
  a.x = x;
  a.x_dtype = x_dtype & kXDtypeMask;
  a.norm = (x_dtype & BITLINEAR_X_RMSNORM) != 0;
  const int per16 = a.x_dtype == BITLINEAR_BF16 ? 8 : 4;
  a.x_vec = (K % per16 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
}

// 16-byte pieces of the activation rows when they are read as pieces, else 0.
int64_t x_pieces(const void* x, int x_dtype, int64_t M, int64_t K) {
  const int per16 = (x_dtype & kXDtypeMask) == BITLINEAR_BF16 ? 8 : 4;
  const bool vec = (K % per16 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  return vec ? M * (K / per16) : 0;
}

}  // namespace

hipError_t launch_gemv_multi(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K, int count,
                             const uint8_t* const* packed, const float* const* beta, const int64_t* N, void* const* y,
                             int y_dtype, bool glu, hipStream_t s) {
  GemvPlan p;
  GemvArgs a;
  if (!make_multi(M, K, count, packed, beta, N, y, y_dtype, glu, false, 0, p, a)) return hipErrorInvalidValue;
  a.q = q;
  a.ldq = ldq;
  a.ds = ds;
  return dispatch(p, a, s);
}

hipError_t launch_decode_multi(const void* x, int x_dtype, int64_t M, int64_t K, int count,
                               const uint8_t* const* packed, const float* const* beta, const int64_t* N,
                               void* const* y, int y_dtype, bool glu, hipStream_t s) {
  GemvPlan p;
  GemvArgs a;
  if (!make_multi(M, K, count, packed, beta, N, y, y_dtype, glu, true, x_pieces(x, x_dtype, M, K), p, a))
    return hipErrorInvalidValue;
  set_x(a, x, x_dtype, K);
  return dispatch(p, a, s);
}

hipError_t launch_decode_rq(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K, int count,
                            const uint8_t* const* packed, const float* const* beta, const int64_t* N, void* const* y,
                            int y_dtype, bool glu, int8_t* next_q, int64_t next_ldq, float* next_ds, bool next_norm,
                            void* ws, hipStream_t s) {
  GemvPlan p;
  GemvArgs a;
  if (!make_multi(M, K, count, packed, beta, N, y, y_dtype, glu, false, 0, p, a)) return hipErrorInvalidValue;
  if (p.NB > 2) {  // the requantizing instantiations cover NB <= 2
    p.NB = 2;
    if (!glu) {
      int g = 0;
      for (int i = 0; i < count; ++i) {
        a.seg[i].g0 = g;
        g += (int)ceil_div(a.seg[i].Nt, 2);
      }
      p.Ng = g;
    }
  }
  a.q = q;
  a.ldq = ldq;
  a.ds = ds;
  a.rq_src = static_cast<const float*>(y[0]);
  a.rq_k = (int)N[0];
  a.rq_norm = next_norm;
  a.rq_q = next_q;
  a.rq_ldq = next_ldq;
  a.rq_ds = next_ds;
  a.rq_cnt = static_cast<uint32_t*>(ws);
  if (p.amode == ALDS_Q) return dispatch_mb_nb<ALDS_Q, false, 0, true>(p, a, s);
  if (p.amode == AGLOBAL) return dispatch_mb_nb<AGLOBAL, false, 0, true>(p, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_b1(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M,
                          int64_t K, const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype,
                          hipStream_t s) {
  const GemvPlan p = make_plan(M, N, K, false, false, M * (ldq / 16), 1);
  GemvArgs a = make_args(p, M, K, N, packed, beta, y, y_dtype, nullptr, 1);
  a.q = q;
  a.ldq = ldq;
  a.ds = ds;
  a.rowsum = rowsum;
  if (p.amode == ALDS_Q) return dispatch_mb_nb<ALDS_Q, false, 1>(p, a, s);
  return dispatch_mb_nb<AGLOBAL, false, 1>(p, a, s);
}

hipError_t launch_gemv_b3(const int8_t* q, int64_t ldq, const float* ds, const int32_t* rowsum, int64_t M,
                          int64_t K, const uint8_t* packed, const float* beta, int64_t N, void* y, int y_dtype,
                          hipStream_t s) {
  const GemvPlan p = make_plan(M, N, K, false, false, M * (ldq / 16), 2);
  GemvArgs a = make_args(p, M, K, N, packed, beta, y, y_dtype, nullptr, 2);
  a.q = q;
  a.ldq = ldq;
  a.ds = ds;
  a.rowsum = rowsum;
  if (p.amode == ALDS_Q) return dispatch_mb_nb<ALDS_Q, false, 2>(p, a, s);
  return dispatch_mb_nb<AGLOBAL, false, 2>(p, a, s);
}

// Token counts for which the small-batch matrix-core path of the prefill
// product (bitlinear_gemm's 32- and 64-row blocks, bit-identical results)
// beats this kernel: from 49 tokens; from 33 on matrices of 2^24 weights or
// more; from 12 on 2^27 or more (measured on the 2B- and 100B-class shapes).
bool gemv_prefers_gemm(int64_t M, int64_t N, int64_t K) {
  if (wide_shape(M, ceil_div(N, kTileN), M * lds_row(K), 0, false)) return false;  // a wide plan
  const int64_t w = N * K;
  return M > 48 || (M > 32 && w >= (int64_t(1) << 24)) || (M >= 12 && w >= (int64_t(1) << 27));
}

int64_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return gemv_prefers_gemm(M, N, K) ? gemm_ws_bytes(M, N, K) : make_plan(M, N, K, false, true, 0, 0, true).ws_bytes;
}

// Host model of the decode kernel's global reads for bitlinear_gemv(_b1,_b3)
// at these sizes (int8 rows of ldq bytes): walks every workgroup, wave and
// k-tile of the kernel's plan, including the ring's clamped re-loads, with the
// kernel's own offset function, and returns one past the last byte any lane
// reads of the activations and of the packed weights.
void gemv_read_extent(int64_t M, int64_t N, int64_t K, int fmt, int64_t ldq, int64_t* act_end, int64_t* w_end) {
  const GemvPlan p = make_plan(M, N, K, false, fmt == 0, M * (ldq / 16), fmt, fmt == 0);
  const int KT = tile_cols(fmt), NS = KT / 64;
  int64_t ae = 0, we = 0;
  for (int grp = 0; grp < p.Ng; ++grp)
    for (int sb = 0; sb < p.SB; ++sb)
      for (int wave = 0; wave < p.waves; ++wave) {
        // the kernel's k-tiles of this wave: kof(s), s < ns
        const int split = sb * p.waves + wave;
        const int kst = p.kint ? p.waves : 1, kb = p.kint ? wave : split * p.tps;
        const int ns = p.kint ? (p.Kt > wave ? (p.Kt - wave + p.waves - 1) / p.waves : 0)
                              : std::max(0, std::min(p.tps, p.Kt - kb));
        // the prologue's unconditional ring loads read kof(0 .. ns - 1) (tile
        // 0 without work); the loop's re-loads are clamped to kof(ns - 1)
        for (int s = 0; s < std::max(ns, 1); ++s) {
          const int kt = ns > 0 ? kb + s * kst : 0;
          for (int j = 0; j < p.NB; ++j) {
            const int64_t nb = std::min(grp * p.NB + j, p.Nt - 1);
            we = std::max(we, (nb * p.Kt + kt) * kTileBytes + kTileBytes);
          }
          if (p.amode != AGLOBAL || ns == 0) continue;
          const int64_t row = std::min<int64_t>(p.MB * 16 - 1, M - 1) * ldq;
          for (int i = 0; i < NS; ++i)
            for (int g4 = 0; g4 < 4; ++g4) ae = std::max(ae, row + act_col(kt, i, g4, KT, ldq, fmt == 2) + 16);
        }
      }
  if (p.amode != AGLOBAL) ae = M * ldq;  // rows staged whole: pieces < M * ldq / 16
  *act_end = ae;
  *w_end = we;
}

bool decode_fused_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= BITLINEAR_GEMV_MAX_M && M * lds_row(K) <= kDecodeLdsBytes;
}

hipError_t launch_gemv_t2(const int8_t* q, int64_t ldq, const float* ds, int64_t M, int64_t K,
                          const uint8_t* packed, const float* beta, int64_t N, void* y,
                          int y_dtype, void* ws, hipStream_t s) {
  if (gemv_prefers_gemm(M, N, K)) return launch_gemm_t2(q, ldq, ds, M, K, packed, beta, N, y, y_dtype, ws, s);
  const GemvPlan p = make_plan(M, N, K, false, true, M * (ldq / 16), 0, true);
  GemvArgs a = make_args(p, M, K, N, packed, beta, y, y_dtype, ws);
  a.q = q;
  a.ldq = ldq;
  a.ds = ds;
  return dispatch(p, a, s);
}

hipError_t launch_decode_t2(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* packed,
                            const float* beta, int64_t N, void* y, int y_dtype, hipStream_t s) {
  const GemvPlan p = make_plan(M, N, K, true, true, x_pieces(x, x_dtype, M, K), 0, true);
  GemvArgs a = make_args(p, M, K, N, packed, beta, y, y_dtype, nullptr);
  set_x(a, x, x_dtype, K);
  return dispatch(p, a, s);
}

}  // namespace bl
