/*
 * bitlinear.h - C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear forward.
 *
 * The operation is the BitLinear layer with ternary weights and 8-bit
 * activations:
 *   - weights: absmean ternarization, beta = mean |W| over the tensor and
 *     T = clamp(round(W / (beta + 1e-8)), -1, 1)
 *     ("Key Technologies Enabling the BitNET Family", Advanced Quantization
 *     Methodologies; "BitNet / Ternary / Binary - Les LLMs 1-bit", Apercu de
 *     l'entrainement d'un BitLinear);
 *   - activations: per-token absmax quantization to int8 (same section of the
 *     first page; Hacker News Reader item 39537919: int8 at inference);
 *   - product: every weight adds, subtracts or skips one activation, summed in
 *     int32 ("BitNet / Ternary / Binary - Les LLMs 1-bit", TL;DR; Hacker News
 *     Reader item 39537919, the reply on summing activations with weight +1
 *     minus those with weight -1);
 *   - output: y = acc * (ds * beta), the inverse of both quantizer scales.
 * The layer shape follows the page's BitLinear(in_features, out_features,
 * bias=False): weights are [N][K] = [out][in], no bias, Y[M][N] = f(X[M][K]).
 *
 * Conventions for every call below
 *   - Pointers to tensors are DEVICE pointers owned by the caller; the library
 *     never frees or keeps them.  They must be 16-byte aligned unless a call
 *     says otherwise.  Tensors are row-major and dense.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     compute call only enqueues work on it and returns; nothing synchronizes
 *     with the host and nothing allocates device memory.
 *   - Every call validates all arguments before enqueuing anything.  On error
 *     it enqueues nothing, returns a negative status and
 *     bitlinear_last_error() (per host thread) says why.  A launch failure
 *     returns BITLINEAR_ERR_HIP.
 *   - M = 0 (no tokens) is a valid no-op.  N = 0 or K = 0 is BITLINEAR_ERR_SHAPE.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified codes.
 *   - Calls are thread-safe.  Calls sharing one workspace must not overlap.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BITLINEAR_OK 0
#define BITLINEAR_ERR_ARG (-1)         /* null pointer, unknown dtype, short workspace */
#define BITLINEAR_ERR_SHAPE (-2)       /* size outside the supported range */
#define BITLINEAR_ERR_ALIGN (-3)       /* pointer not aligned as required */
#define BITLINEAR_ERR_UNSUPPORTED (-4) /* valid request this build does not implement */
#define BITLINEAR_ERR_HIP (-5)         /* the HIP runtime reported an error */

/* Element types. */
#define BITLINEAR_F32 0  /* IEEE fp32 */
#define BITLINEAR_BF16 1 /* bfloat16, round-to-nearest-even when written */
#define BITLINEAR_I32 2  /* raw int32 accumulators (output only) */
#define BITLINEAR_F32_ADD 3 /* fp32, added to what y holds: y += value (output only) */

/* Flag OR-ed into an activation x_dtype: RMS-normalize each token row (gain
 * 1, no bias) before it is quantized ("Key Technologies Enabling the BitNET
 * Family", Architectural Innovations and Optimizations: RMSNorm is the
 * normalization).  S = sum_k x_k^2 in fp64, r = 1 / sqrt((float)(S / K) +
 * 1e-5) in fp32, and the quantizer sees fl(x_k * r); x_ds then refers to the
 * normalized row.  The fp64 sum is taken in a fixed but unspecified order. */
#define BITLINEAR_X_RMSNORM 16

/* Supported sizes. */
#define BITLINEAR_MAX_K 131072       /* keeps 64 * 127 * K below 2^31 */
#define BITLINEAR_MAX_N 1048576
#define BITLINEAR_MAX_M 1048576
#define BITLINEAR_GEMV_MAX_M 64

/* Library version, (major << 16) | minor. */
int bitlinear_version(void);

/* Last error message of the calling host thread; never NULL. */
const char *bitlinear_last_error(void);

/*
 * Bytes per row of the int8 activation buffer x_q: K rounded up to a multiple
 * of 512 (the columns of a binary weight tile).  Entries k >= K of each row
 * are written as 0 by bitlinear_quant_act and must stay 0.  Returns -1 for K
 * outside [1, BITLINEAR_MAX_K].
 */
int64_t bitlinear_act_stride(int64_t K);

/*
 * Size in bytes of the packed ternary weights for an N x K matrix:
 * ceil(N/16) * ceil(K/256) * 1024 (2 bits per weight, padded to whole tiles).
 * Returns -1 for N or K outside the supported range.
 */
int64_t bitlinear_packed_bytes(int64_t N, int64_t K);

/*
 * Size in bytes of packed binary weights (bitlinear_pack_weights_b1) for an
 * N x K matrix: ceil(N/16) * ceil(K/512) * 1024 (1 bit per weight, padded to
 * whole tiles).  Returns -1 for N or K outside the supported range.
 */
int64_t bitlinear_packed_bytes_b1(int64_t N, int64_t K);

/* Workspace bytes bitlinear_pack_weights(_b1) needs: 8 * ceil(N*K / 4096). */
int64_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);

/*
 * Workspace bytes bitlinear_gemv / bitlinear_gemm need for this shape (may be
 * 0): int32 partial sums when the k-range of a product is split across
 * workgroups (few output columns with a long K for bitlinear_gemv; up to 64
 * tokens with few output blocks for bitlinear_gemm, which bitlinear_gemv also
 * uses for its larger batches).  A workspace must be filled with zeros once
 * before its first use; every call that returns BITLINEAR_OK leaves it filled
 * with zeros again.  Calls that share a workspace must not run concurrently.
 */
int64_t bitlinear_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K);
int64_t bitlinear_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Introspection for tests (no GPU needed, computes nothing on a device): the
 * read extents of the decode product kernel that bitlinear_gemv (format 0),
 * bitlinear_gemv_b1 (1) or bitlinear_gemv_b3 (2) launches for M tokens, K
 * inputs and N outputs, modelled on the host from the kernel's own plan and
 * offset arithmetic.  *act_end is one past the last byte of x_q (rows of
 * bitlinear_act_stride(K) bytes) any lane reads, *w_end one past the last
 * byte of the packed weights.  Both must stay within M * act_stride(K) and
 * the packed size.  (For format 0, bitlinear_gemv hands larger batches to
 * the prefill kernel; the model describes the decode kernel's plan.)
 * Returns BITLINEAR_ERR_SHAPE for M outside [1, BITLINEAR_GEMV_MAX_M] or N, K
 * out of range, BITLINEAR_ERR_ARG for an unknown format or a null pointer.
 */
int bitlinear_gemv_read_extent(int64_t M, int64_t N, int64_t K, int format, int64_t *act_end,
                               int64_t *w_end);

/*
 * Per-token absmax activation quantization ("Key Technologies Enabling the
 * BitNET Family", Advanced Quantization Methodologies: 8-bit activations,
 * absmax, per token; Hacker News Reader item 39537919: activations are int8 at
 * inference).
 *   x        [M][K] activations, x_dtype BITLINEAR_BF16 or BITLINEAR_F32,
 *            optionally | BITLINEAR_X_RMSNORM;
 *            needs only element alignment (2 or 4 bytes).
 *   x_q      [M][bitlinear_act_stride(K)] int8 out:
 *            q = clamp(rint(x * (127 / g)), -127, 127), g = max(max_k |x|, 1e-5),
 *            rint = round half to even; padding columns are written as 0.
 *   x_ds     [M] fp32 out: g / 127 (the dequantization factor of the token).
 *   x_rowsum [M] int32 out, sum_k q (may be NULL).
 * Errors: ERR_ARG (null x/x_q/x_ds, unknown dtype), ERR_SHAPE (K or M out of
 * range), ERR_ALIGN (x_q not 16-byte aligned, x not element aligned).
 */
int bitlinear_quant_act(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *x_q,
                        float *x_ds, int32_t *x_rowsum, void *stream);

/*
 * Absmean ternarization and 2-bit packing of latent fp32 weights ("BitNet /
 * Ternary / Binary - Les LLMs 1-bit", Apercu de l'entrainement d'un BitLinear:
 * beta = mean |w|, clamp(round(w / (beta + 1e-8)), -1, 1); "BitNet Technical
 * Notes", Appendix glossary: 2 bits per ternary weight).
 *   w         [N][K] fp32 latent weights (4-byte aligned).
 *   packed    bitlinear_packed_bytes(N, K) bytes out, the tiled 2-bit format:
 *             tile (nb, kb) of 16 rows x 256 columns is 1024 bytes at byte
 *             offset (nb * ceil(K/256) + kb) * 1024; byte 16*L + 4*d + b of the
 *             tile holds in bits 2i..2i+1 the code of weight
 *             (n = 16*nb + L%16, k = 256*kb + 64*i + 16*(L/16) + 4*d + b),
 *             code +1 -> 01, 0 -> 00, -1 -> 11; padding holds 00.
 *   w_beta    [1] fp32 out: beta = mean |w|, summed in fp64 in a fixed order
 *             (chunks of 4096 consecutive elements in row-major order, each
 *             summed in index order, chunk sums added in ascending order) and
 *             rounded once to fp32.  Codes use d = beta + 1e-8 (fp32),
 *             t = clamp(rint(w / d), -1, 1).
 *   workspace bitlinear_pack_workspace_bytes(N, K) bytes of scratch (8-byte
 *             aligned; contents on entry do not matter).
 * Errors: ERR_ARG (null pointer), ERR_SHAPE (N or K out of range), ERR_ALIGN.
 */
int bitlinear_pack_weights(const float *w, int64_t N, int64_t K, void *packed, float *w_beta,
                           void *workspace, void *stream);

/*
 * Ternary matrix product with dequantization, for few tokens (decode): every
 * weight adds, subtracts or skips one int8 activation ("BitNet / Ternary /
 * Binary - Les LLMs 1-bit", TL;DR; Hacker News Reader item 39537919, the reply
 * on summing activations with weight +1 minus those with weight -1), the int32
 * sum rescaled by both quantizer scales.
 *   x_q, x_ds  output of bitlinear_quant_act for M tokens and K inputs.
 *   packed, w_beta  output of bitlinear_pack_weights for N x K weights.
 *   y          [M][N] out, y_dtype BITLINEAR_F32 (y = acc * (ds * beta) in
 *              fp32), BITLINEAR_BF16 (the same value rounded to nearest even)
 *              or BITLINEAR_I32 (the raw accumulator acc = sum_k q * t),
 *              or BITLINEAR_F32_ADD (y = y + acc * (ds * beta), two fp32
 *              roundings: the residual sum of a decoder layer fused into
 *              the product; y must not overlap x_q or x_ds).
 *              Needs element alignment only.
 *   workspace  bitlinear_gemv_workspace_bytes(M, N, K) bytes (NULL if 0).
 * M must be in [0, BITLINEAR_GEMV_MAX_M].
 * Errors: ERR_ARG, ERR_SHAPE, ERR_ALIGN as above.
 */
int bitlinear_gemv(const int8_t *x_q, const float *x_ds, int64_t M, int64_t K, const void *packed,
                   const float *w_beta, int64_t N, void *y, int y_dtype, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * The same product for any number of tokens (prefill), on the int8 matrix
 * cores (same passages as bitlinear_gemv: at many tokens the add / subtract /
 * skip sum is a dense contraction).  Arguments as bitlinear_gemv; M in
 * [0, BITLINEAR_MAX_M].
 */
int bitlinear_gemm(const int8_t *x_q, const float *x_ds, int64_t M, int64_t K, const void *packed,
                   const float *w_beta, int64_t N, void *y, int y_dtype, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Binary weights, BitNet b1 ("BitNet / Ternary / Binary - Les LLMs 1-bit",
 * TL;DR and Mecanisme technique: every weight is exactly +1 or -1).
 * bitlinear_pack_weights_b1: t = +1 where w >= 0, else -1 (the pages give no
 * rule; zero maps to +1), beta as bitlinear_pack_weights; packed holds
 * bitlinear_packed_bytes_b1(N, K) bytes: tile (nb, kb) of 16 rows x 512
 * columns is 1024 bytes at offset (nb * ceil(K/512) + kb) * 1024; 32-bit word
 * d of lane L (bytes 16*L + 4*d, little endian) holds in bit 16*h + j the
 * weight (n = 16*nb + L%16, k = 512*kb + 64*(2*d + h) + 16*(L/16) + j),
 * bit 1 = +1, bit 0 = -1; padding bits are 0.  Errors as bitlinear_pack_weights.
 */
int bitlinear_pack_weights_b1(const float *w, int64_t N, int64_t K, void *packed, float *w_beta,
                              void *workspace, void *stream);

/*
 * Binary-weight product for few tokens: y = dequant(acc), acc[m][n] =
 * sum_k q[m][k] * t[n][k] with t in {-1, +1}, dequantized exactly as
 * bitlinear_gemv.  x_rowsum [M] int32 (required): the row sums written by
 * bitlinear_quant_act for the same x_q.  Other arguments as bitlinear_gemv;
 * uses no workspace.  M in [0, BITLINEAR_GEMV_MAX_M].
 * Errors: ERR_ARG (null pointer, x_rowsum missing), ERR_SHAPE, ERR_ALIGN.
 */
int bitlinear_gemv_b1(const int8_t *x_q, const float *x_ds, const int32_t *x_rowsum, int64_t M,
                      int64_t K, const void *packed, const float *w_beta, int64_t N, void *y,
                      int y_dtype, void *stream);

/* The same binary-weight product for any number of tokens (prefill), on the
 * int8 matrix cores.  Arguments as bitlinear_gemv_b1; M in [0, BITLINEAR_MAX_M]. */
int bitlinear_gemm_b1(const int8_t *x_q, const float *x_ds, const int32_t *x_rowsum, int64_t M,
                      int64_t K, const void *packed, const float *w_beta, int64_t N, void *y,
                      int y_dtype, void *stream);

/*
 * Base-3 packing of the ternary weights, five to a byte (1.6 bits per
 * weight; "BitNet Technical Notes" and the "BitNet: Inference framework for
 * 1-bit LLMs" thread discuss packing trits more densely than 2 bits).
 * bitlinear_packed_bytes_b3(N, K) = ceil(N/16) * ceil(K/320) * 1024.
 * bitlinear_pack_weights_b3: the same beta and codes t as
 * bitlinear_pack_weights, stored as tiles (nb, kb) of 16 rows x 320 columns,
 * 1024 bytes at offset (nb * ceil(K/320) + kb) * 1024; byte 16*L + i of a tile
 * (L in 0..63, i in 0..15) is sum_{s=0..4} (t + 1) * 3^s over the weights
 * (n = 16*nb + L%16, k = 320*kb + 64*s + 16*(L/16) + i); padding adds 0.
 * bitlinear_gemv_b3: the decode product on those tiles, identical to
 * bitlinear_gemv on the same weights; x_rowsum [M] int32 is required (from
 * bitlinear_quant_act).  Arguments and errors as bitlinear_gemv_b1.
 */
int64_t bitlinear_packed_bytes_b3(int64_t N, int64_t K);
int bitlinear_pack_weights_b3(const float *w, int64_t N, int64_t K, void *packed, float *w_beta,
                              void *workspace, void *stream);
int bitlinear_gemv_b3(const int8_t *x_q, const float *x_ds, const int32_t *x_rowsum, int64_t M,
                      int64_t K, const void *packed, const float *w_beta, int64_t N, void *y,
                      int y_dtype, void *stream);

/*
 * Training step of a BitLinear with the straight-through estimator ("BitNet /
 * Ternary / Binary - Les LLMs 1-bit", Apercu de l'entrainement d'un
 * BitLinear): the forward uses the quantized weights, the backward passes the
 * gradient to the latent weights unchanged.  Activations and gradients are
 * bf16 and not quantized; the weights enter as beta * t from
 * bitlinear_pack_weights (packed, w_beta).  fp32 accumulation on the bf16
 * matrix cores, fp32 outputs (row-major, 4-byte aligned):
 *   bitlinear_train_forward:         y  [M][N] = beta * x . t^T,  x  [M][K]
 *   bitlinear_train_backward_input:  dx [M][K] = beta * dy . t,   dy [M][N]
 *   bitlinear_train_backward_weight: dw [N][K] = dy^T . x
 * bf16 inputs need 2-byte alignment (16-byte rows run faster).  M, N, K in
 * [0 or 1, the BITLINEAR_MAX_* limits]; M = 0 writes nothing.
 * Errors: ERR_ARG (null pointer), ERR_SHAPE, ERR_ALIGN.
 */
int bitlinear_train_forward(const void *x, int64_t M, int64_t K, const void *packed, const float *w_beta,
                            int64_t N, float *y, void *stream);
int bitlinear_train_backward_input(const void *dy, int64_t M, int64_t N, const void *packed,
                                   const float *w_beta, int64_t K, float *dx, void *stream);
int bitlinear_train_backward_weight(const void *dy, const void *x, int64_t M, int64_t N, int64_t K,
                                    float *dw, void *stream);

/* LDS budget of the decode kernels for int8 activation rows (see below). */
#define BITLINEAR_DECODE_MAX_ACT_BYTES 58368

/*
 * Whole BitLinear forward for decode, in one launch: per-token absmax int8
 * quantization of x (as bitlinear_quant_act) fused into the ternary product
 * with dequantization (as bitlinear_gemv).  Each workgroup quantizes the
 * token rows into its own LDS, so no int8 buffer is written.  Results are
 * identical to bitlinear_quant_act followed by bitlinear_gemv.  Every
 * workgroup quantizes the whole rows again, so this pays off for few tokens
 * (measured on MI355X: M <= 4); beyond that the two calls are faster.
 *   x       [M][K] activations, x_dtype BITLINEAR_BF16 or BITLINEAR_F32,
 *           optionally | BITLINEAR_X_RMSNORM (element alignment).
 *   packed, w_beta, y, y_dtype  as bitlinear_gemv.
 * Needs M * (K rounded up to 256, + 16) <= BITLINEAR_DECODE_MAX_ACT_BYTES,
 * else BITLINEAR_ERR_UNSUPPORTED (use bitlinear_quant_act + bitlinear_gemv).
 * Other errors as bitlinear_gemv.  Uses no workspace.
 */
int bitlinear_forward_decode(const void *x, int x_dtype, int64_t M, int64_t K, const void *packed,
                             const float *w_beta, int64_t N, void *y, int y_dtype, void *stream);

/* Most BitLinears one multi call computes. */
#define BITLINEAR_MULTI_MAX 4

/*
 * Several BitLinears that read the same activations, in one launch (e.g. the
 * q, k and v projections of a decoder layer): y_i = dequant(x_q . T_i^T) for
 * i < count, each exactly as bitlinear_gemv would compute it.
 *   count     1 .. BITLINEAR_MULTI_MAX.
 *   packed, w_beta, N, y  host arrays of count entries (read during the call
 *             only), each entry as the single-matrix argument of
 *             bitlinear_gemv; all outputs share y_dtype.
 * Uses no workspace.  M in [0, BITLINEAR_GEMV_MAX_M].
 * Errors: ERR_ARG (null array or entry, count out of range), ERR_SHAPE,
 * ERR_ALIGN, as bitlinear_gemv for every entry.
 */
int bitlinear_gemv_multi(const int8_t *x_q, const float *x_ds, int64_t M, int64_t K, int count,
                         const void *const *packed, const float *const *w_beta, const int64_t *N,
                         void *const *y, int y_dtype, void *stream);

/* The same with the activation quantization fused (as bitlinear_forward_decode). */
int bitlinear_forward_decode_multi(const void *x, int x_dtype, int64_t M, int64_t K, int count,
                                   const void *const *packed, const float *const *w_beta,
                                   const int64_t *N, void *const *y, int y_dtype, void *stream);

/*
 * Gated feed-forward pair in one launch ("Key Technologies Enabling the BitNET
 * Family", Architectural Innovations and Optimizations: squared ReLU in the
 * feed-forward layers): with g = BL_gate(x), u = BL_up(x) (both N x K,
 * dequantized to fp32 exactly as bitlinear_gemv),
 *   h[m][n] = (r * r) * u[m][n],  r = g[m][n] if g[m][n] > 0 else +0,
 * identical to two products followed by bitlinear_relu2_mul; g and u are
 * never written.  h [M][N] fp32 device output, 4-byte aligned.
 * Errors as bitlinear_gemv.  Uses no workspace.
 */
int bitlinear_gemv_glu(const int8_t *x_q, const float *x_ds, int64_t M, int64_t K,
                       const void *packed_gate, const float *beta_gate, const void *packed_up,
                       const float *beta_up, int64_t N, float *h, void *stream);

/* The same with the activation quantization fused (as bitlinear_forward_decode). */
int bitlinear_forward_decode_glu(const void *x, int x_dtype, int64_t M, int64_t K,
                                 const void *packed_gate, const float *beta_gate,
                                 const void *packed_up, const float *beta_up, int64_t N, float *h,
                                 void *stream);

/*
 * Decode product with the next BitLinear's activation quantization in its
 * epilogue ("Key Technologies Enabling the BitNET Family", Advanced
 * Quantization Methodologies: the next layer's input is quantized per token
 * by absmax; Architectural Innovations and Optimizations: RMSNorm before it).
 * The same products as bitlinear_gemv_multi (glu = 0: count 1 .. 4
 * BitLinears sharing x_q) or bitlinear_gemv_glu (glu = 1: count 2, packed[0]
 * the gate and packed[1] the up matrix, y[0] receives h); then the last
 * workgroup to finish quantizes the M fp32 rows of y[0] (or h), RMS-normalized
 * first when next_flags is BITLINEAR_X_RMSNORM, into next_q
 * [M][bitlinear_act_stride(N[0])] and next_ds [M], with the arithmetic of
 * bitlinear_quant_act(y[0], BITLINEAR_F32 | next_flags): identical codes and
 * scales, except that the fp64 sum of squares of the normalization is taken
 * in another fixed order (its last bits can differ, which changes the fp32
 * mean square only at an fp32 rounding boundary).
 * This saves the quantizer's launch between two BitLinears of a decode step.
 *   y_dtype    for glu = 0: BITLINEAR_F32 or BITLINEAR_F32_ADD (the residual
 *              sum, y[0] += ...); y[0] is 16-byte aligned.
 *   next_q     16-byte aligned, must not overlap x_q, y or h.
 *   workspace  16 bytes, 16-byte aligned, zero before the first call; every
 *              successful call leaves it zero (an arrival counter).  Calls
 *              sharing a workspace must not overlap.
 * Errors: as bitlinear_gemv_multi / bitlinear_gemv_glu, and ERR_ARG for
 * next_flags, a non-fp32 y_dtype, or a short workspace.
 */
int bitlinear_decode_rq(const int8_t *x_q, const float *x_ds, int64_t M, int64_t K, int count, int glu,
                        const void *const *packed, const float *const *w_beta, const int64_t *N,
                        void *const *y, int y_dtype, int8_t *next_q, float *next_ds, int next_flags,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Feed-forward activation between the gate / up and down BitLinears of a
 * decoder layer ("Key Technologies Enabling the BitNET Family", Architectural
 * Innovations and Optimizations: squared ReLU in the feed-forward layers):
 *   h[i] = (r * r) * u[i],  r = g[i] if g[i] > 0 else +0,
 * fp32, two roundings in this order.
 *   g, u     [count] fp32 device inputs (gate and up projections).
 *   h        [count] fp32 device output; may be g or u (elementwise).
 * All pointers 4-byte aligned; count == 0 enqueues nothing.
 * Errors: ERR_ARG (null pointer), ERR_SHAPE (count < 0), ERR_ALIGN.
 */
int bitlinear_relu2_mul(const float *g, const float *u, int64_t count, float *h, void *stream);

/* Bytes of the device array bitlinear_gemv_noalloc uses as scratch. */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES (8 << 20)

/*
 * bitlinear_gemv for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same product, arguments and results as bitlinear_gemv, but the split-k
 * partial sums some shapes need live in a fixed array of
 * BITLINEAR_NOALLOC_SCRATCH_BYTES in device memory that each GPU holds until
 * the process ends, instead of a caller-provided workspace.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * the caller still passes inputs and outputs.  Every shape bitlinear_gemv
 * accepts needs at most 8 MiB (bitlinear_gemv_workspace_bytes); a shape
 * needing more would return BITLINEAR_ERR_UNSUPPORTED.  The array is shared
 * by every call on the same GPU and keeps the last call's contents (zero
 * after each successful call; cleared by a kernel on first use and after a
 * failed launch): calls that overlap on one GPU race and must be serialized,
 * e.g. on one stream.
 * Errors: as bitlinear_gemv.
 */
int bitlinear_gemv_noalloc(const int8_t *x_q, const float *x_ds, int64_t M, int64_t K,
                           const void *packed, const float *w_beta, int64_t N, void *y, int y_dtype,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
