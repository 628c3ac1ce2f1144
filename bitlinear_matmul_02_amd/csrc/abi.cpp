// C ABI of libbitlinear: argument validation, error reporting, dispatch.
// Nothing here touches the GPU before every argument has been checked, so an
// invalid call enqueues nothing (and works without a GPU present).
#include <stdarg.h>
#include <stdio.h>

#include "bl_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return BITLINEAR_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BITLINEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool k_ok(int64_t K) { return K >= 1 && K <= BITLINEAR_MAX_K; }
bool n_ok(int64_t N) { return N >= 1 && N <= BITLINEAR_MAX_N; }

int64_t act_stride(int64_t K) { return bl::ceil_div(K, bl::kActAlign) * bl::kActAlign; }

// Activation rows the fused decode kernels stage in LDS: K rounded up to 256, + 16.
int64_t fused_row(int64_t K) { return bl::ceil_div(K, bl::kTileK) * bl::kTileK + 16; }

// Shape, dtype and weight/output checks shared by every product call.
int check_common(const char* fn, int64_t M, int64_t max_m, int64_t K, const void* packed, const float* w_beta,
                 int64_t N, void* y, int y_dtype) {
  if (M < 0 || M > max_m) return fail(BITLINEAR_ERR_SHAPE, "%s: M=%lld outside [0, %lld]", fn, (long long)M, (long long)max_m);
  if (!k_ok(K)) return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld outside [1, %d]", fn, (long long)K, BITLINEAR_MAX_K);
  if (!n_ok(N)) return fail(BITLINEAR_ERR_SHAPE, "%s: N=%lld outside [1, %d]", fn, (long long)N, BITLINEAR_MAX_N);
  if (y_dtype != BITLINEAR_F32 && y_dtype != BITLINEAR_BF16 && y_dtype != BITLINEAR_I32 &&
      y_dtype != BITLINEAR_F32_ADD)
    return fail(BITLINEAR_ERR_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
  if (M == 0) return BITLINEAR_OK;
  if (!packed || !w_beta || !y) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(packed, 16)) return fail(BITLINEAR_ERR_ALIGN, "%s: packed must be 16-byte aligned", fn);
  if (!aligned(w_beta, 4) || !aligned(y, y_dtype == BITLINEAR_BF16 ? 2 : 4))
    return fail(BITLINEAR_ERR_ALIGN, "%s: w_beta or y not element aligned", fn);
  return BITLINEAR_OK;
}

// Checks of gemv / gemm: the common ones, the int8 activations, the workspace.
int check_product(const char* fn, const int8_t* x_q, const float* x_ds, int64_t M, int64_t max_m,
                  int64_t K, const void* packed, const float* w_beta, int64_t N, void* y,
                  int y_dtype, void* ws, size_t ws_bytes, int64_t need_ws) {
  int st = check_common(fn, M, max_m, K, packed, w_beta, N, y, y_dtype);
  if (st != BITLINEAR_OK || M == 0) return st;
  if (!x_q || !x_ds) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(x_q, 16)) return fail(BITLINEAR_ERR_ALIGN, "%s: x_q must be 16-byte aligned", fn);
  if (!aligned(x_ds, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: x_ds not element aligned", fn);
  if (need_ws > 0) {
    if (!ws) return fail(BITLINEAR_ERR_ARG, "%s: this shape needs a %lld-byte workspace", fn, (long long)need_ws);
    if ((int64_t)ws_bytes < need_ws)
      return fail(BITLINEAR_ERR_ARG, "%s: workspace of %zu bytes, %lld needed", fn, ws_bytes, (long long)need_ws);
    if (!aligned(ws, 16)) return fail(BITLINEAR_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  }
  return BITLINEAR_OK;
}

}  // namespace

extern "C" {

int bitlinear_version(void) { return (1 << 16) | 3; }

const char* bitlinear_last_error(void) { return g_err; }

int64_t bitlinear_act_stride(int64_t K) { return k_ok(K) ? act_stride(K) : -1; }

int64_t bitlinear_packed_bytes(int64_t N, int64_t K) {
  if (!n_ok(N) || !k_ok(K)) return -1;
  return bl::ceil_div(N, bl::kTileN) * bl::ceil_div(K, bl::kTileK) * bl::kTileBytes;
}

int64_t bitlinear_packed_bytes_b1(int64_t N, int64_t K) {
  if (!n_ok(N) || !k_ok(K)) return -1;
  return bl::ceil_div(N, bl::kTileN) * bl::ceil_div(K, bl::kTileKB1) * bl::kTileBytes;
}

int64_t bitlinear_packed_bytes_b3(int64_t N, int64_t K) {
  if (!n_ok(N) || !k_ok(K)) return -1;
  return bl::ceil_div(N, bl::kTileN) * bl::ceil_div(K, bl::kTileKB3) * bl::kTileBytes;
}

int64_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K) {
  if (!n_ok(N) || !k_ok(K)) return -1;
  return 8 * bl::ceil_div(N * K, bl::kBetaChunk);
}

int64_t bitlinear_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || M > BITLINEAR_GEMV_MAX_M || !n_ok(N) || !k_ok(K)) return -1;
  return M == 0 ? 0 : bl::gemv_ws_bytes(M, N, K);
}

int64_t bitlinear_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || M > BITLINEAR_MAX_M || !n_ok(N) || !k_ok(K)) return -1;
  return M == 0 ? 0 : bl::gemm_ws_bytes(M, N, K);
}

int bitlinear_gemv_read_extent(int64_t M, int64_t N, int64_t K, int format, int64_t* act_end, int64_t* w_end) {
  const char* fn = "bitlinear_gemv_read_extent";
  if (M < 1 || M > BITLINEAR_GEMV_MAX_M || !n_ok(N) || !k_ok(K))
    return fail(BITLINEAR_ERR_SHAPE, "%s: M=%lld, N=%lld, K=%lld out of range", fn, (long long)M, (long long)N,
                (long long)K);
  if (format < 0 || format > 2) return fail(BITLINEAR_ERR_ARG, "%s: unknown format %d", fn, format);
  if (!act_end || !w_end) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  bl::gemv_read_extent(M, N, K, format, act_stride(K), act_end, w_end);
  return ok();
}

int bitlinear_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* x_q, float* x_ds,
                        int32_t* x_rowsum, void* stream) {
  const char* fn = "bitlinear_quant_act";
  const int x_base = x_dtype & ~BITLINEAR_X_RMSNORM;
  if (x_base != BITLINEAR_BF16 && x_base != BITLINEAR_F32)
    return fail(BITLINEAR_ERR_ARG, "%s: x_dtype must be BITLINEAR_BF16 or BITLINEAR_F32 (| BITLINEAR_X_RMSNORM)", fn);
  if (M < 0 || M > BITLINEAR_MAX_M) return fail(BITLINEAR_ERR_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
  if (!k_ok(K)) return fail(BITLINEAR_ERR_SHAPE, "%s: K=%lld outside [1, %d]", fn, (long long)K, BITLINEAR_MAX_K);
  if (M == 0) return ok();
  if (!x || !x_q || !x_ds) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(x, x_base == BITLINEAR_BF16 ? 2 : 4) || !aligned(x_q, 16) || !aligned(x_ds, 4) ||
      (x_rowsum && !aligned(x_rowsum, 4)))
    return fail(BITLINEAR_ERR_ALIGN, "%s: misaligned pointer (x_q needs 16 bytes)", fn);
  return hip_status(bl::launch_quant_act(x, x_dtype, M, K, act_stride(K), x_q, x_ds, x_rowsum,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_pack_weights(const float* w, int64_t N, int64_t K, void* packed, float* w_beta,
                           void* workspace, void* stream) {
  const char* fn = "bitlinear_pack_weights";
  if (!n_ok(N) || !k_ok(K))
    return fail(BITLINEAR_ERR_SHAPE, "%s: N=%lld, K=%lld out of range", fn, (long long)N, (long long)K);
  if (!w || !packed || !w_beta || !workspace) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(w, 4) || !aligned(packed, 16) || !aligned(w_beta, 4) || !aligned(workspace, 8))
    return fail(BITLINEAR_ERR_ALIGN, "%s: misaligned pointer", fn);
  return hip_status(bl::launch_pack_t2(w, N, K, static_cast<uint8_t*>(packed), w_beta,
                                       static_cast<double*>(workspace), static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_pack_weights_b1(const float* w, int64_t N, int64_t K, void* packed, float* w_beta, void* workspace,
                              void* stream) {
  const char* fn = "bitlinear_pack_weights_b1";
  if (!n_ok(N) || !k_ok(K))
    return fail(BITLINEAR_ERR_SHAPE, "%s: N=%lld or K=%lld out of range", fn, (long long)N, (long long)K);
  if (!w || !packed || !w_beta || !workspace) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(w, 4) || !aligned(packed, 16) || !aligned(w_beta, 4) || !aligned(workspace, 8))
    return fail(BITLINEAR_ERR_ALIGN, "%s: misaligned pointer", fn);
  return hip_status(bl::launch_pack_b1(w, N, K, static_cast<uint8_t*>(packed), w_beta, static_cast<double*>(workspace),
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_pack_weights_b3(const float* w, int64_t N, int64_t K, void* packed, float* w_beta, void* workspace,
                              void* stream) {
  const char* fn = "bitlinear_pack_weights_b3";
  if (!n_ok(N) || !k_ok(K))
    return fail(BITLINEAR_ERR_SHAPE, "%s: N=%lld or K=%lld out of range", fn, (long long)N, (long long)K);
  if (!w || !packed || !w_beta || !workspace) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(w, 4) || !aligned(packed, 16) || !aligned(w_beta, 4) || !aligned(workspace, 8))
    return fail(BITLINEAR_ERR_ALIGN, "%s: misaligned pointer", fn);
  return hip_status(bl::launch_pack_b3(w, N, K, static_cast<uint8_t*>(packed), w_beta, static_cast<double*>(workspace),
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_gemv(const int8_t* x_q, const float* x_ds, int64_t M, int64_t K, const void* packed,
                   const float* w_beta, int64_t N, void* y, int y_dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const char* fn = "bitlinear_gemv";
  const int64_t need = (M >= 1 && M <= BITLINEAR_GEMV_MAX_M && n_ok(N) && k_ok(K)) ? bl::gemv_ws_bytes(M, N, K) : 0;
  int st = check_product(fn, x_q, x_ds, M, BITLINEAR_GEMV_MAX_M, K, packed, w_beta, N, y, y_dtype,
                         workspace, workspace_bytes, need);
  if (st != BITLINEAR_OK || M == 0) return st == BITLINEAR_OK ? ok() : st;
  return hip_status(bl::launch_gemv_t2(x_q, act_stride(K), x_ds, M, K, static_cast<const uint8_t*>(packed),
                                       w_beta, N, y, y_dtype, workspace, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_gemv_noalloc(const int8_t* x_q, const float* x_ds, int64_t M, int64_t K, const void* packed,
                           const float* w_beta, int64_t N, void* y, int y_dtype, void* stream) {
  const char* fn = "bitlinear_gemv_noalloc";
  int st = check_product(fn, x_q, x_ds, M, BITLINEAR_GEMV_MAX_M, K, packed, w_beta, N, y, y_dtype, nullptr, 0, 0);
  if (st != BITLINEAR_OK || M == 0) return st == BITLINEAR_OK ? ok() : st;
  const int64_t need = bl::gemv_ws_bytes(M, N, K);
  if (need > BITLINEAR_NOALLOC_SCRATCH_BYTES)
    return fail(BITLINEAR_ERR_UNSUPPORTED, "%s: this shape needs %lld bytes of scratch, more than the %d-byte device "
                "array; use bitlinear_gemv with a workspace", fn, (long long)need, BITLINEAR_NOALLOC_SCRATCH_BYTES);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = bl::noalloc_scratch(s, &ws);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  const hipError_t e = bl::launch_gemv_t2(x_q, act_stride(K), x_ds, M, K, static_cast<const uint8_t*>(packed), w_beta,
                                          N, y, y_dtype, ws, s);
  if (e != hipSuccess && need > 0) bl::noalloc_mark_dirty();
  return hip_status(e, fn);
}

int bitlinear_gemm(const int8_t* x_q, const float* x_ds, int64_t M, int64_t K, const void* packed,
                   const float* w_beta, int64_t N, void* y, int y_dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const char* fn = "bitlinear_gemm";
  const int64_t need = (M >= 1 && M <= BITLINEAR_MAX_M && n_ok(N) && k_ok(K)) ? bl::gemm_ws_bytes(M, N, K) : 0;
  int st = check_product(fn, x_q, x_ds, M, BITLINEAR_MAX_M, K, packed, w_beta, N, y, y_dtype,
                         workspace, workspace_bytes, need);
  if (st != BITLINEAR_OK || M == 0) return st == BITLINEAR_OK ? ok() : st;
  return hip_status(bl::launch_gemm_t2(x_q, act_stride(K), x_ds, M, K, static_cast<const uint8_t*>(packed),
                                       w_beta, N, y, y_dtype, workspace, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_gemv_b1(const int8_t* x_q, const float* x_ds, const int32_t* x_rowsum, int64_t M, int64_t K,
                      const void* packed, const float* w_beta, int64_t N, void* y, int y_dtype, void* stream) {
  const char* fn = "bitlinear_gemv_b1";
  int st = check_product(fn, x_q, x_ds, M, BITLINEAR_GEMV_MAX_M, K, packed, w_beta, N, y, y_dtype, nullptr, 0, 0);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  if (!x_rowsum) return fail(BITLINEAR_ERR_ARG, "%s: x_rowsum is required", fn);
  if (!aligned(x_rowsum, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: x_rowsum not element aligned", fn);
  return hip_status(bl::launch_gemv_b1(x_q, act_stride(K), x_ds, x_rowsum, M, K, static_cast<const uint8_t*>(packed),
                                       w_beta, N, y, y_dtype, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_gemv_b3(const int8_t* x_q, const float* x_ds, const int32_t* x_rowsum, int64_t M, int64_t K,
                      const void* packed, const float* w_beta, int64_t N, void* y, int y_dtype, void* stream) {
  const char* fn = "bitlinear_gemv_b3";
  int st = check_product(fn, x_q, x_ds, M, BITLINEAR_GEMV_MAX_M, K, packed, w_beta, N, y, y_dtype, nullptr, 0, 0);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  if (!x_rowsum) return fail(BITLINEAR_ERR_ARG, "%s: x_rowsum is required", fn);
  if (!aligned(x_rowsum, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: x_rowsum not element aligned", fn);
  return hip_status(bl::launch_gemv_b3(x_q, act_stride(K), x_ds, x_rowsum, M, K, static_cast<const uint8_t*>(packed),
                                       w_beta, N, y, y_dtype, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_gemm_b1(const int8_t* x_q, const float* x_ds, const int32_t* x_rowsum, int64_t M, int64_t K,
                      const void* packed, const float* w_beta, int64_t N, void* y, int y_dtype, void* stream) {
  const char* fn = "bitlinear_gemm_b1";
  int st = check_product(fn, x_q, x_ds, M, BITLINEAR_MAX_M, K, packed, w_beta, N, y, y_dtype, nullptr, 0, 0);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  if (!x_rowsum) return fail(BITLINEAR_ERR_ARG, "%s: x_rowsum is required", fn);
  if (!aligned(x_rowsum, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: x_rowsum not element aligned", fn);
  return hip_status(bl::launch_gemm_b1(x_q, act_stride(K), x_ds, x_rowsum, M, K, static_cast<const uint8_t*>(packed),
                                       w_beta, N, y, y_dtype, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_forward_decode(const void* x, int x_dtype, int64_t M, int64_t K, const void* packed,
                             const float* w_beta, int64_t N, void* y, int y_dtype, void* stream) {
  const char* fn = "bitlinear_forward_decode";
  const int x_base = x_dtype & ~BITLINEAR_X_RMSNORM;
  if (x_base != BITLINEAR_BF16 && x_base != BITLINEAR_F32)
    return fail(BITLINEAR_ERR_ARG, "%s: x_dtype must be BITLINEAR_BF16 or BITLINEAR_F32 (| BITLINEAR_X_RMSNORM)", fn);
  int st = check_common(fn, M, BITLINEAR_GEMV_MAX_M, K, packed, w_beta, N, y, y_dtype);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  if (!x) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(x, x_base == BITLINEAR_BF16 ? 2 : 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: x not element aligned", fn);
  if (!bl::decode_fused_fits(M, K))
    return fail(BITLINEAR_ERR_UNSUPPORTED, "%s: M * (K rounded up to 256 + 16) = %lld exceeds %d bytes", fn,
                (long long)(M * fused_row(K)), BITLINEAR_DECODE_MAX_ACT_BYTES);
  return hip_status(bl::launch_decode_t2(x, x_dtype, M, K, static_cast<const uint8_t*>(packed), w_beta, N, y,
                                         y_dtype, static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"

namespace {

// Checks of one multi / gated call; x_q/x_ds (product) or x (fused) are
// checked by the caller.
int check_multi(const char* fn, int64_t M, int64_t K, int count, const void* const* packed,
                const float* const* w_beta, const int64_t* N, void* const* y, int y_dtype) {
  if (!packed || !w_beta || !N || !y) return fail(BITLINEAR_ERR_ARG, "%s: null array argument", fn);
  if (count < 1 || count > BITLINEAR_MULTI_MAX)
    return fail(BITLINEAR_ERR_ARG, "%s: count %d outside [1, %d]", fn, count, BITLINEAR_MULTI_MAX);
  for (int i = 0; i < count; ++i) {
    int st = check_common(fn, M, BITLINEAR_GEMV_MAX_M, K, packed[i], w_beta[i], N[i], y[i], y_dtype);
    if (st != BITLINEAR_OK) return st;
  }
  return BITLINEAR_OK;
}

int check_x(const char* fn, const void* x, int x_dtype, int64_t M, int64_t K) {
  const int x_base = x_dtype & ~BITLINEAR_X_RMSNORM;
  if (x_base != BITLINEAR_BF16 && x_base != BITLINEAR_F32)
    return fail(BITLINEAR_ERR_ARG, "%s: x_dtype must be BITLINEAR_BF16 or BITLINEAR_F32 (| BITLINEAR_X_RMSNORM)", fn);
  if (M == 0) return BITLINEAR_OK;
  if (!x) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(x, x_base == BITLINEAR_BF16 ? 2 : 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: x not element aligned", fn);
  if (!bl::decode_fused_fits(M, K))
    return fail(BITLINEAR_ERR_UNSUPPORTED, "%s: M * (K rounded up to 256 + 16) = %lld exceeds %d bytes", fn,
                (long long)(M * fused_row(K)), BITLINEAR_DECODE_MAX_ACT_BYTES);
  return BITLINEAR_OK;
}

int check_q(const char* fn, const int8_t* x_q, const float* x_ds, int64_t M) {
  if (M == 0) return BITLINEAR_OK;
  if (!x_q || !x_ds) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(x_q, 16) || !aligned(x_ds, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: x_q must be 16-byte aligned", fn);
  return BITLINEAR_OK;
}

const uint8_t* const* as_bytes(const void* const* p) { return reinterpret_cast<const uint8_t* const*>(p); }

}  // namespace

extern "C" {

int bitlinear_gemv_multi(const int8_t* x_q, const float* x_ds, int64_t M, int64_t K, int count,
                         const void* const* packed, const float* const* w_beta, const int64_t* N, void* const* y,
                         int y_dtype, void* stream) {
  const char* fn = "bitlinear_gemv_multi";
  int st = check_multi(fn, M, K, count, packed, w_beta, N, y, y_dtype);
  if (st == BITLINEAR_OK) st = check_q(fn, x_q, x_ds, M);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  return hip_status(bl::launch_gemv_multi(x_q, act_stride(K), x_ds, M, K, count, as_bytes(packed), w_beta, N, y,
                                          y_dtype, false, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_forward_decode_multi(const void* x, int x_dtype, int64_t M, int64_t K, int count,
                                   const void* const* packed, const float* const* w_beta, const int64_t* N,
                                   void* const* y, int y_dtype, void* stream) {
  const char* fn = "bitlinear_forward_decode_multi";
  int st = check_multi(fn, M, K, count, packed, w_beta, N, y, y_dtype);
  if (st == BITLINEAR_OK) st = check_x(fn, x, x_dtype, M, K);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  return hip_status(bl::launch_decode_multi(x, x_dtype, M, K, count, as_bytes(packed), w_beta, N, y, y_dtype,
                                            false, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_decode_rq(const int8_t* x_q, const float* x_ds, int64_t M, int64_t K, int count, int glu,
                        const void* const* packed, const float* const* w_beta, const int64_t* N, void* const* y,
                        int y_dtype, int8_t* next_q, float* next_ds, int next_flags, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const char* fn = "bitlinear_decode_rq";
  if (glu != 0 && glu != 1) return fail(BITLINEAR_ERR_ARG, "%s: glu must be 0 or 1", fn);
  if (glu && count != 2) return fail(BITLINEAR_ERR_ARG, "%s: a gated pair has count 2", fn);
  if (next_flags != 0 && next_flags != BITLINEAR_X_RMSNORM)
    return fail(BITLINEAR_ERR_ARG, "%s: next_flags must be 0 or BITLINEAR_X_RMSNORM", fn);
  if (!glu && y_dtype != BITLINEAR_F32 && y_dtype != BITLINEAR_F32_ADD)
    return fail(BITLINEAR_ERR_ARG, "%s: the requantized output must be fp32 (BITLINEAR_F32 or BITLINEAR_F32_ADD)", fn);
  void* hy[2] = {nullptr, nullptr};
  if (glu) {
    if (!y || !y[0]) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
    hy[0] = hy[1] = y[0];
  }
  int st = check_multi(fn, M, K, count, packed, w_beta, N, glu ? hy : y, glu ? BITLINEAR_F32 : y_dtype);
  if (st == BITLINEAR_OK && glu && N[0] != N[1]) st = fail(BITLINEAR_ERR_SHAPE, "%s: gate and up differ in N", fn);
  if (st == BITLINEAR_OK) st = check_q(fn, x_q, x_ds, M);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  if (!next_q || !next_ds || !workspace) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(next_q, 16) || !aligned(next_ds, 4) || !aligned(workspace, 16) || !aligned(y[0], 16))
    return fail(BITLINEAR_ERR_ALIGN, "%s: next_q, workspace and y[0] must be 16-byte aligned, next_ds 4-byte", fn);
  if (workspace_bytes < 16) return fail(BITLINEAR_ERR_ARG, "%s: workspace of %zu bytes, 16 needed", fn, workspace_bytes);
  return hip_status(bl::launch_decode_rq(x_q, act_stride(K), x_ds, M, K, count, as_bytes(packed), w_beta, N,
                                         glu ? hy : y, glu ? BITLINEAR_F32 : y_dtype, glu != 0, next_q,
                                         act_stride(N[0]), next_ds, next_flags != 0, workspace,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_gemv_glu(const int8_t* x_q, const float* x_ds, int64_t M, int64_t K, const void* packed_gate,
                       const float* beta_gate, const void* packed_up, const float* beta_up, int64_t N, float* h,
                       void* stream) {
  const char* fn = "bitlinear_gemv_glu";
  const void* packed[2] = {packed_gate, packed_up};
  const float* beta[2] = {beta_gate, beta_up};
  const int64_t n2[2] = {N, N};
  void* y[2] = {h, h};
  int st = check_multi(fn, M, K, 2, packed, beta, n2, y, BITLINEAR_F32);
  if (st == BITLINEAR_OK) st = check_q(fn, x_q, x_ds, M);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  return hip_status(bl::launch_gemv_multi(x_q, act_stride(K), x_ds, M, K, 2, as_bytes(packed), beta, n2, y,
                                          BITLINEAR_F32, true, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_forward_decode_glu(const void* x, int x_dtype, int64_t M, int64_t K, const void* packed_gate,
                                 const float* beta_gate, const void* packed_up, const float* beta_up, int64_t N,
                                 float* h, void* stream) {
  const char* fn = "bitlinear_forward_decode_glu";
  const void* packed[2] = {packed_gate, packed_up};
  const float* beta[2] = {beta_gate, beta_up};
  const int64_t n2[2] = {N, N};
  void* y[2] = {h, h};
  int st = check_multi(fn, M, K, 2, packed, beta, n2, y, BITLINEAR_F32);
  if (st == BITLINEAR_OK) st = check_x(fn, x, x_dtype, M, K);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  return hip_status(bl::launch_decode_multi(x, x_dtype, M, K, 2, as_bytes(packed), beta, n2, y, BITLINEAR_F32,
                                            true, static_cast<hipStream_t>(stream)),
                    fn);
}

// Shapes and pointers of the training products (M rows of activations).
static int check_train(const char* fn, int64_t M, int64_t N, int64_t K, const void* p0, const void* p1,
                       const void* p2, const void* out) {
  if (M < 0 || M > BITLINEAR_MAX_M) return fail(BITLINEAR_ERR_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
  if (!n_ok(N) || !k_ok(K))
    return fail(BITLINEAR_ERR_SHAPE, "%s: N=%lld or K=%lld out of range", fn, (long long)N, (long long)K);
  if (M == 0) return BITLINEAR_OK;
  if (!p0 || !p1 || !p2 || !out) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(out, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: output not 4-byte aligned", fn);
  return BITLINEAR_OK;
}

int bitlinear_train_forward(const void* x, int64_t M, int64_t K, const void* packed, const float* w_beta, int64_t N,
                            float* y, void* stream) {
  const char* fn = "bitlinear_train_forward";
  int st = check_train(fn, M, N, K, x, packed, w_beta, y);
  if (st != BITLINEAR_OK || M == 0) return st == BITLINEAR_OK ? ok() : st;
  if (!aligned(x, 2) || !aligned(packed, 16) || !aligned(w_beta, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: misaligned input", fn);
  return hip_status(bl::launch_train_forward(static_cast<const uint16_t*>(x), M, K, static_cast<const uint8_t*>(packed),
                                             w_beta, N, y, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_train_backward_input(const void* dy, int64_t M, int64_t N, const void* packed, const float* w_beta,
                                   int64_t K, float* dx, void* stream) {
  const char* fn = "bitlinear_train_backward_input";
  int st = check_train(fn, M, N, K, dy, packed, w_beta, dx);
  if (st != BITLINEAR_OK || M == 0) return st == BITLINEAR_OK ? ok() : st;
  if (!aligned(dy, 2) || !aligned(packed, 16) || !aligned(w_beta, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: misaligned input", fn);
  return hip_status(bl::launch_train_dx(static_cast<const uint16_t*>(dy), M, N, static_cast<const uint8_t*>(packed),
                                        w_beta, K, dx, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_train_backward_weight(const void* dy, const void* x, int64_t M, int64_t N, int64_t K, float* dw,
                                    void* stream) {
  const char* fn = "bitlinear_train_backward_weight";
  int st = check_train(fn, M, N, K, dy, x, x, dw);
  if (st != BITLINEAR_OK) return st;
  if (M == 0) return ok();
  if (!aligned(dy, 2) || !aligned(x, 2)) return fail(BITLINEAR_ERR_ALIGN, "%s: misaligned input", fn);
  return hip_status(bl::launch_train_dw(static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(x), M, N, K,
                                        dw, static_cast<hipStream_t>(stream)),
                    fn);
}

int bitlinear_relu2_mul(const float* g, const float* u, int64_t count, float* h, void* stream) {
  const char* fn = "bitlinear_relu2_mul";
  if (count < 0) return fail(BITLINEAR_ERR_SHAPE, "%s: count %lld < 0", fn, (long long)count);
  if (count == 0) return ok();
  if (!g || !u || !h) return fail(BITLINEAR_ERR_ARG, "%s: null pointer argument", fn);
  if (!aligned(g, 4) || !aligned(u, 4) || !aligned(h, 4)) return fail(BITLINEAR_ERR_ALIGN, "%s: pointers must be 4-byte aligned", fn);
  return hip_status(bl::launch_relu2_mul(g, u, count, h, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
