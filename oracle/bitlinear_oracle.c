/*
 * Plain CPU oracle for the BitNet b1.58 BitLinear forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) never calls it and shares no code, header, table or helper
 * with it; both sides are written independently from the method's definition
 * and from the packed-format specification.
 *
 * Everything here is the plain definition written out: straight loops, no
 * intrinsics, no blocking, no fusion.  Built with -ffp-contract=off and no
 * fast-math, so every float operation below is one IEEE-754 operation in
 * round-to-nearest-even, in the order written.
 *
 * What each function follows (page title, then section):
 *  - oracle_absmean, oracle_ternarize:
 *      "Key Technologies Enabling the BitNET Family", Advanced Quantization
 *      Methodologies (absmean ternary weights);
 *      "BitNet / Ternary / Binary - Les LLMs 1-bit", Apercu de l'entrainement
 *      d'un BitLinear (beta = mean |w|; clamp(round(w / (beta + 1e-8)), -1, 1)).
 *  - oracle_quant_act:
 *      "Key Technologies Enabling the BitNET Family", Advanced Quantization
 *      Methodologies (8-bit activations, absmax, per token); Hacker News
 *      Reader item 39537919 (activations are int8 at inference).
 *  - oracle_matmul_i32:
 *      "BitNet / Ternary / Binary - Les LLMs 1-bit", TL;DR and Mecanisme
 *      technique (products become add / subtract / skip); Hacker News Reader
 *      item 39537919, the reply that corrects the "elementwise additions"
 *      wording (sum of activations with weight +1 minus those with weight -1).
 *  - oracle_dequant_f32, oracle_f32_to_bf16: rescaling by the two quantizer
 *      scales; implied by the quantizer pair above, not printed on the pages.
 *  - oracle_rmsnorm_f32: RMS normalization of each token row before it is
 *      quantized (same page and section as the squared ReLU below: RMSNorm
 *      is the normalization, without bias terms).
 *  - oracle_relu2_mul, oracle_add_f32: the decoder glue around the
 *      BitLinears of one layer ("Key Technologies Enabling the BitNET
 *      Family", Architectural Innovations and Optimizations: squared ReLU in
 *      the feed-forward layers); the residual sums of a decoder layer.
 *  - oracle_binarize, oracle_pack_b1 / oracle_unpack_b1: the binary
 *      variant BitNet b1 ("BitNet / Ternary / Binary - Les LLMs 1-bit",
 *      TL;DR and Mecanisme technique: every weight is exactly +1 or -1), one
 *      bit per weight; its layout is this project's own choice, written here
 *      from its specification.
 *  - oracle_pack_b3 / oracle_unpack_b3: ternary weights five to a byte in
 *      base 3 (1.6 bits per weight; "BitNet Technical Notes" and the
 *      "BitNet: Inference framework for 1-bit LLMs" thread discuss packing
 *      trits more densely than 2 bits); the layout is this project's own
 *      choice, written here from its specification.
 *  - oracle_train_forward / oracle_train_dx / oracle_train_dw: the training
 *      step of a BitLinear with the straight-through estimator ("BitNet /
 *      Ternary / Binary - Les LLMs 1-bit", Apercu de l'entrainement d'un
 *      BitLinear: the forward multiplies by the quantized weights, the
 *      backward lets the gradient pass to the latent weights unchanged).
 *  - oracle_pack_t2 / oracle_unpack_t2: 2 bits per ternary weight
 *      ("BitNet Technical Notes", Appendix glossary: bit-packing at 2 bits per
 *      ternary weight; "BitNet: Inference framework for 1-bit LLMs", post #139:
 *      two bits hold a spare fourth value).  The bit layout itself is this
 *      project's own choice and is written here from its specification.
 *
 * Readings where the pages are silent (each stated in the design notes):
 *  - beta: mean |w| in fp64, summed in a fixed order (consecutive chunks of
 *    4096 elements in row-major order, each chunk summed in index order, the
 *    chunk sums added in ascending chunk order), then rounded once to fp32.
 *  - binary weights (the pages give no binarization rule): t = +1 where
 *    w >= 0, else -1 (so zero maps to +1 and the set stays {-1, +1}); the
 *    scale is the same beta = mean |w| as for the ternary weights.
 *  - rounding: half to even (torch.round semantics, the IEEE default).
 *  - activations: gamma = max |x|; g = max(gamma, 1e-5); q = clamp(rint(x *
 *    (127 / g)), -127, 127); ds = g / 127.
 *  - dequant: y = (float)acc * (ds * beta).
 *  - RMS normalization (gain 1, no bias; placement and epsilon not given on
 *    the pages): S = sum_k x_k^2 in fp64 (each square exact), ms = (float)(S /
 *    K), r = 1 / sqrt(ms + 1e-5) in fp32, xn_k = x_k * r.
 *  - training products: bf16 inputs (activations and output gradients are not
 *    quantized, as in the pages' training snippet), the quantized weights
 *    scaled by beta (as at inference; the snippet omits the rescale):
 *    y = x . (beta t)^T, dx = dy . (beta t), dw = dy^T . x, each sum exact in
 *    fp64, times beta in fp64, rounded once to fp32.
 *  - feed-forward glue: h = (r * r) * u with r = g if g > 0 else 0, fp32 in
 *    this order; the gate / up / down form is the plainest reading of an FFN
 *    with ReLU^2 between its projections.
 *
 * Parity status: every function here is pinned by the CPU test suite
 * (hand-worked example, brute force, closed forms, invariants, the pages'
 * popcount forms); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BETA_CHUNK 4096
#define ORACLE_EPS_W 1e-8f
#define ORACLE_EPS_X 1e-5f
#define ORACLE_EPS_NORM 1e-5f

/* ---------------------------------------------------------------- weights */

/* beta = mean |w| over the whole tensor (per-tensor, no grouping). */
float oracle_absmean(const float *w, int64_t count)
{
    double total = 0.0;
    for (int64_t c0 = 0; c0 < count; c0 += ORACLE_BETA_CHUNK) {
        int64_t c1 = c0 + ORACLE_BETA_CHUNK;
        if (c1 > count)
            c1 = count;
        double part = 0.0;
        for (int64_t i = c0; i < c1; ++i)
            part += fabs((double)w[i]);
        total += part;
    }
    return (float)(total / (double)count);
}

/* t = clamp(round_half_even(w / (beta + 1e-8)), -1, 1), elementwise. */
void oracle_ternarize(const float *w, int64_t count, float beta, int8_t *t)
{
    float d = beta + ORACLE_EPS_W;
    for (int64_t i = 0; i < count; ++i) {
        float r = rintf(w[i] / d);
        if (r > 1.0f)
            r = 1.0f;
        if (r < -1.0f)
            r = -1.0f;
        t[i] = (int8_t)r;
    }
}

/* ------------------------------------------------------------ activations */

static float bf16_bits_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static void quant_row(const float *x, int64_t K, int8_t *q, float *ds, int32_t *rowsum)
{
    float gamma = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = fabsf(x[k]);
        if (a > gamma)
            gamma = a;
    }
    float g = gamma > ORACLE_EPS_X ? gamma : ORACLE_EPS_X;
    float qs = 127.0f / g;
    int32_t s = 0;
    for (int64_t k = 0; k < K; ++k) {
        float v = rintf(x[k] * qs);
        if (v > 127.0f)
            v = 127.0f;
        if (v < -127.0f)
            v = -127.0f;
        q[k] = (int8_t)v;
        s += q[k];
    }
    *ds = g / 127.0f;
    *rowsum = s;
}

/* Per-token absmax int8 quantization of fp32 activations x[M][K]. */
void oracle_quant_act_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *ds,
                          int32_t *rowsum)
{
    for (int64_t m = 0; m < M; ++m)
        quant_row(x + m * K, K, q + m * K, ds + m, rowsum + m);
}

/* Same, for activations given as bf16 bit patterns (converted exactly). */
void oracle_quant_act_bf16(const uint16_t *xb, int64_t M, int64_t K, int8_t *q, float *ds,
                           int32_t *rowsum)
{
    float *row = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
    if (!row)
        return;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            row[k] = bf16_bits_to_f32(xb[m * K + k]);
        quant_row(row, K, q + m * K, ds + m, rowsum + m);
    }
    free(row);
}

/* -------------------------------------------------------------- products */

/* acc[m][n] = sum_k q[m][k] * t[n][k]   (naive triple loop, exact int32).
 * threads > 1 splits the n loop over OpenMP threads (timing only; the
 * result does not depend on it). */
void oracle_matmul_i32(const int8_t *q, const int8_t *t, int64_t M, int64_t N, int64_t K,
                       int32_t *acc, int threads)
{
    if (threads < 1)
        threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int32_t)q[m * K + k] * (int32_t)t[n * K + k];
            acc[m * N + n] = s;
        }
}

/* The same sums for a list of (m, n) pairs only (large shapes, sampled). */
void oracle_matmul_i32_pairs(const int8_t *q, const int8_t *t, int64_t K, const int64_t *ms,
                             const int64_t *ns, int64_t count, int32_t *out)
{
    for (int64_t p = 0; p < count; ++p) {
        const int8_t *qa = q + ms[p] * K;
        const int8_t *ta = t + ns[p] * K;
        int32_t s = 0;
        for (int64_t k = 0; k < K; ++k)
            s += (int32_t)qa[k] * (int32_t)ta[k];
        out[p] = s;
    }
}

/* y[m][n] = (float)acc[m][n] * (ds[m] * beta). */
void oracle_dequant_f32(const int32_t *acc, const float *ds, float beta, int64_t M, int64_t N,
                        float *y)
{
    for (int64_t m = 0; m < M; ++m) {
        float s = ds[m] * beta;
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (float)acc[m * N + n] * s;
    }
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even. */
void oracle_f32_to_bf16(const float *y, int64_t count, uint16_t *out)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t u;
        memcpy(&u, &y[i], sizeof u);
        if ((u & 0x7fffffffu) > 0x7f800000u) { /* NaN: keep it a quiet NaN */
            out[i] = (uint16_t)((u >> 16) | 0x0040u);
            continue;
        }
        uint32_t lower = u & 0xffffu;
        uint32_t upper = u >> 16;
        if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
            upper += 1u;
        out[i] = (uint16_t)upper;
    }
}

/* ------------------------------------------------------- packed formats
 *
 * Format T2 (2 bits per weight).  Weights W[N][K] are cut into tiles of
 * 16 rows x 256 columns; tile (nb, kb) is 1024 bytes at byte offset
 * (nb * ceil(K/256) + kb) * 1024.  Inside a tile, byte 16*L + 4*d + b
 * (L in 0..63, d in 0..3, b in 0..3) holds four 2-bit fields; field i
 * (bits 2i and 2i+1) is the code of weight
 *     n = 16*nb + (L mod 16),
 *     k = 256*kb + 64*i + 16*(L div 16) + 4*d + b.
 * Code: +1 -> 01, 0 -> 00, -1 -> 11 (two's complement of t in two bits);
 * 10 is never written.  Positions with n >= N or k >= K hold 00.
 */
int64_t oracle_t2_bytes(int64_t N, int64_t K)
{
    return ((N + 15) / 16) * ((K + 255) / 256) * 1024;
}

void oracle_pack_t2(const int8_t *t, int64_t N, int64_t K, uint8_t *packed)
{
    int64_t Kt = (K + 255) / 256;
    memset(packed, 0, (size_t)oracle_t2_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t nb = n / 16, kb = k / 256;
            int64_t r = n % 16, c = k % 256;
            int64_t i = c / 64, g = (c % 64) / 16, d = (c % 16) / 4, b = c % 4;
            int64_t L = 16 * g + r;
            int64_t byte = (nb * Kt + kb) * 1024 + 16 * L + 4 * d + b;
            uint8_t code = (uint8_t)(t[n * K + k] & 3);
            packed[byte] |= (uint8_t)(code << (2 * i));
        }
}

/* Inverse of oracle_pack_t2.  Returns the number of fields holding the
 * never-written code 10 (0 for a well-formed buffer); such fields decode
 * as 0 here. */
int64_t oracle_unpack_t2(const uint8_t *packed, int64_t N, int64_t K, int8_t *t)
{
    int64_t Kt = (K + 255) / 256, bad = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t nb = n / 16, kb = k / 256;
            int64_t r = n % 16, c = k % 256;
            int64_t i = c / 64, g = (c % 64) / 16, d = (c % 16) / 4, b = c % 4;
            int64_t L = 16 * g + r;
            int64_t byte = (nb * Kt + kb) * 1024 + 16 * L + 4 * d + b;
            int code = (packed[byte] >> (2 * i)) & 3;
            if (code == 1)
                t[n * K + k] = 1;
            else if (code == 3)
                t[n * K + k] = -1;
            else {
                if (code == 2)
                    ++bad;
                t[n * K + k] = 0;
            }
        }
    return bad;
}

/*
 * Format B1 (1 bit per weight).  Tiles of 16 rows x 512 columns; tile
 * (nb, kb) is 1024 bytes at byte offset (nb * ceil(K/512) + kb) * 1024.
 * Inside a tile, 32-bit word d of lane L (bytes 16*L + 4*d .. +3, little
 * endian; L in 0..63, d in 0..3) holds in bit 16*h + j (h in 0..1, j in
 * 0..15) the weight
 *     n = 16*nb + (L mod 16),
 *     k = 512*kb + 64*(2*d + h) + 16*(L div 16) + j.
 * Bit 1 is +1, bit 0 is -1.  Positions with n >= N or k >= K hold 0.
 */
int64_t oracle_b1_bytes(int64_t N, int64_t K)
{
    return ((N + 15) / 16) * ((K + 511) / 512) * 1024;
}

/* t = +1 where w >= 0, else -1 */
void oracle_binarize(const float *w, int64_t count, int8_t *t)
{
    for (int64_t i = 0; i < count; ++i)
        t[i] = w[i] >= 0.0f ? 1 : -1;
}

void oracle_pack_b1(const int8_t *t, int64_t N, int64_t K, uint8_t *packed)
{
    int64_t Kt = (K + 511) / 512;
    memset(packed, 0, (size_t)oracle_b1_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            if (t[n * K + k] != 1)
                continue;
            int64_t nb = n / 16, kb = k / 512;
            int64_t r = n % 16, c = k % 512;
            int64_t s = c / 64, g = (c % 64) / 16, j = c % 16;
            int64_t L = 16 * g + r, d = s / 2, h = s % 2;
            int64_t bit = 16 * h + j;
            int64_t byte = (nb * Kt + kb) * 1024 + 16 * L + 4 * d + bit / 8;
            packed[byte] |= (uint8_t)(1u << (bit % 8));
        }
}

/* Inverse of oracle_pack_b1 over the N x K weights. */
void oracle_unpack_b1(const uint8_t *packed, int64_t N, int64_t K, int8_t *t)
{
    int64_t Kt = (K + 511) / 512;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t nb = n / 16, kb = k / 512;
            int64_t r = n % 16, c = k % 512;
            int64_t s = c / 64, g = (c % 64) / 16, j = c % 16;
            int64_t L = 16 * g + r, d = s / 2, h = s % 2;
            int64_t bit = 16 * h + j;
            int64_t byte = (nb * Kt + kb) * 1024 + 16 * L + 4 * d + bit / 8;
            t[n * K + k] = (packed[byte] >> (bit % 8)) & 1 ? 1 : -1;
        }
}

/*
 * Format B3 (five ternary weights per byte, base 3).  Tiles of 16 rows x 320
 * columns; tile (nb, kb) is 1024 bytes at byte offset (nb * ceil(K/320) + kb)
 * * 1024.  Byte 16*L + i of a tile (L in 0..63, i in 0..15) is
 *     sum_{s=0..4} c_s * 3^s,  c_s = t(n, k_s) + 1 in {0, 1, 2},
 *     n = 16*nb + (L mod 16),  k_s = 320*kb + 64*s + 16*(L div 16) + i.
 * Positions with n >= N or k >= K contribute c = 0.
 */
int64_t oracle_b3_bytes(int64_t N, int64_t K)
{
    return ((N + 15) / 16) * ((K + 319) / 320) * 1024;
}

void oracle_pack_b3(const int8_t *t, int64_t N, int64_t K, uint8_t *packed)
{
    static const int pow3[5] = {1, 3, 9, 27, 81};
    int64_t Kt = (K + 319) / 320;
    memset(packed, 0, (size_t)oracle_b3_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t nb = n / 16, kb = k / 320;
            int64_t r = n % 16, c = k % 320;
            int64_t s = c / 64, g = (c % 64) / 16, i = c % 16;
            int64_t L = 16 * g + r;
            int64_t byte = (nb * Kt + kb) * 1024 + 16 * L + i;
            packed[byte] = (uint8_t)(packed[byte] + (t[n * K + k] + 1) * pow3[s]);
        }
}

/* Inverse of oracle_pack_b3 over the N x K weights. */
void oracle_unpack_b3(const uint8_t *packed, int64_t N, int64_t K, int8_t *t)
{
    int64_t Kt = (K + 319) / 320;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t nb = n / 16, kb = k / 320;
            int64_t r = n % 16, c = k % 320;
            int64_t s = c / 64, g = (c % 64) / 16, i = c % 16;
            int64_t L = 16 * g + r;
            int v = packed[(nb * Kt + kb) * 1024 + 16 * L + i];
            for (int64_t j = 0; j < s; ++j)
                v /= 3;
            t[n * K + k] = (int8_t)(v % 3 - 1);
        }
}

/* ------------------------------------------------------- decoder glue */

/* h = ReLU(g)^2 * u elementwise: r = g if g > 0 else +0, then (r * r) * u,
 * two fp32 roundings in this order. */
void oracle_relu2_mul(const float *g, const float *u, int64_t count, float *h)
{
    for (int64_t i = 0; i < count; ++i) {
        float r = g[i] > 0.0f ? g[i] : 0.0f;
        float r2 = r * r;
        h[i] = r2 * u[i];
    }
}

/* Residual sum x += r, one fp32 rounding per element. */
void oracle_add_f32(float *x, const float *r, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        x[i] = x[i] + r[i];
}

/* RMS normalization of each row of x[M][K] (gain 1): xn = x * r with
 * r = 1 / sqrt(mean(x^2) + eps); the mean of squares is summed in fp64 in
 * index order and rounded once to fp32. */
void oracle_rmsnorm_f32(const float *x, int64_t M, int64_t K, float *xn)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += (double)row[k] * (double)row[k];
        float ms = (float)(s / (double)K);
        float r = 1.0f / sqrtf(ms + ORACLE_EPS_NORM);
        for (int64_t k = 0; k < K; ++k)
            xn[m * K + k] = row[k] * r;
    }
}

/* ------------------------------------------------------------ training */

/* y[m][n] = beta * sum_k x[m][k] t[n][k]  (x bf16 [M][K], t [N][K]) */
void oracle_train_forward(const uint16_t *xb, int64_t M, int64_t K, const int8_t *t, float beta, int64_t N,
                          float *y, int threads)
{
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += (double)bf16_bits_to_f32(xb[m * K + k]) * (double)t[n * K + k];
            y[m * N + n] = (float)((double)beta * s);
        }
}

/* dx[m][k] = beta * sum_n dy[m][n] t[n][k]  (dy bf16 [M][N]) */
void oracle_train_dx(const uint16_t *dyb, int64_t M, int64_t N, const int8_t *t, float beta, int64_t K,
                     float *dx, int threads)
{
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                s += (double)bf16_bits_to_f32(dyb[m * N + n]) * (double)t[n * K + k];
            dx[m * K + k] = (float)((double)beta * s);
        }
}

/* dw[n][k] = sum_m dy[m][n] x[m][k]: the straight-through gradient of the
 * latent weights (dy bf16 [M][N], x bf16 [M][K]) */
void oracle_train_dw(const uint16_t *dyb, const uint16_t *xb, int64_t M, int64_t N, int64_t K, float *dw,
                     int threads)
{
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m)
                s += (double)bf16_bits_to_f32(dyb[m * N + n]) * (double)bf16_bits_to_f32(xb[m * K + k]);
            dw[n * K + k] = (float)s;
        }
}
