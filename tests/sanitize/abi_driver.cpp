// Drives the validation path of every compute entry point of libbitlinear and
// every compute-free helper, for a host build of the library's sources with
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every compute call below
// has at least one invalid argument, so it must return its error status
// before anything reaches a GPU (none is needed); the M = 0 calls are valid
// no-ops.  Pointers are host buffers standing in for device memory: the
// validation only inspects their values.  Exit status 0: every check passed.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <thread>

#include "bitlinear.h"

static int failures = 0;
#define EXPECT(call, code)                                                                                    \
  do {                                                                                                        \
    const int st_ = (call);                                                                                   \
    if (st_ != (code)) {                                                                                      \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, st_, (int)(code),       \
              bitlinear_last_error());                                                                        \
      ++failures;                                                                                             \
    } else if ((code) != BITLINEAR_OK && bitlinear_last_error()[0] == '\0') {                                 \
      fprintf(stderr, "line %d: %s left no error message\n", __LINE__, #call);                                \
      ++failures;                                                                                             \
    }                                                                                                         \
  } while (0)
#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "line %d: %s failed\n", __LINE__, #cond); \
      ++failures;                                              \
    }                                                          \
  } while (0)

int main() {
  alignas(256) static unsigned char buf[1 << 16];
  void* p = buf;                     // aligned stand-in pointer
  void* odd = buf + 1;               // misaligned one
  const int8_t* q = (const int8_t*)p;
  const float* f = (const float*)p;
  float* fo = (float*)p;
  const int32_t* rs = (const int32_t*)p;
  const int bf = BITLINEAR_BF16, f32 = BITLINEAR_F32;

  // helpers
  CHECK(bitlinear_version() > 0);
  CHECK(bitlinear_act_stride(1) == 512 && bitlinear_act_stride(513) == 1024);
  CHECK(bitlinear_act_stride(0) == -1 && bitlinear_act_stride(BITLINEAR_MAX_K + 1) == -1);
  CHECK(bitlinear_packed_bytes(16, 256) == 1024 && bitlinear_packed_bytes(17, 257) == 4096);
  CHECK(bitlinear_packed_bytes(0, 1) == -1 && bitlinear_packed_bytes(1, -5) == -1);
  CHECK(bitlinear_packed_bytes(BITLINEAR_MAX_N, BITLINEAR_MAX_K) > 0);
  CHECK(bitlinear_packed_bytes_b1(BITLINEAR_MAX_N, BITLINEAR_MAX_K) > 0);
  CHECK(bitlinear_packed_bytes_b3(BITLINEAR_MAX_N, BITLINEAR_MAX_K) > 0);
  CHECK(bitlinear_pack_workspace_bytes(BITLINEAR_MAX_N, BITLINEAR_MAX_K) > 0);
  CHECK(bitlinear_pack_workspace_bytes(-1, 4) == -1);
  CHECK(bitlinear_gemv_workspace_bytes(65, 16, 256) == -1);
  CHECK(bitlinear_gemm_workspace_bytes(-1, 16, 256) == -1);
  static const int64_t ms[] = {1, 2, 8, 12, 16, 17, 32, 33, 48, 49, 64};
  static const int64_t nk[][2] = {{1, 1}, {16, 256}, {2560, 6912}, {28672, 8192}, {8192, 28672},
                                  {BITLINEAR_MAX_N, 512}, {16, BITLINEAR_MAX_K}, {300, 7}};
  for (int64_t m : ms)
    for (auto& s : nk) {
      CHECK(bitlinear_gemv_workspace_bytes(m, s[0], s[1]) >= 0);
      CHECK(bitlinear_gemm_workspace_bytes(m, s[0], s[1]) >= 0);
      for (int fmt = 0; fmt < 3; ++fmt) {
        int64_t ae = 0, we = 0;
        if (s[0] * s[1] > (int64_t)1 << 28) continue;  // keep the walk short
        EXPECT(bitlinear_gemv_read_extent(m, s[0], s[1], fmt, &ae, &we), BITLINEAR_OK);
        const int64_t wb = fmt == 0   ? bitlinear_packed_bytes(s[0], s[1])
                           : fmt == 1 ? bitlinear_packed_bytes_b1(s[0], s[1])
                                      : bitlinear_packed_bytes_b3(s[0], s[1]);
        CHECK(ae > 0 && ae <= m * bitlinear_act_stride(s[1]) && we > 0 && we <= wb);
      }
    }
  CHECK(bitlinear_gemm_workspace_bytes(BITLINEAR_MAX_M, BITLINEAR_MAX_N, BITLINEAR_MAX_K) >= 0);

  // quant_act
  EXPECT(bitlinear_quant_act(p, 7, 1, 16, (int8_t*)p, fo, nullptr, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_quant_act(p, bf, -1, 16, (int8_t*)p, fo, nullptr, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_quant_act(p, bf, 1, 0, (int8_t*)p, fo, nullptr, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_quant_act(nullptr, bf, 1, 16, (int8_t*)p, fo, nullptr, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_quant_act(p, bf, 1, 16, (int8_t*)odd, fo, nullptr, nullptr), BITLINEAR_ERR_ALIGN);
  EXPECT(bitlinear_quant_act(odd, f32, 1, 16, (int8_t*)p, fo, nullptr, nullptr), BITLINEAR_ERR_ALIGN);
  EXPECT(bitlinear_quant_act(p, bf | BITLINEAR_X_RMSNORM, 0, 16, nullptr, nullptr, nullptr, nullptr), BITLINEAR_OK);

  // packers
  EXPECT(bitlinear_pack_weights(f, 0, 16, p, fo, p, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_pack_weights(f, 16, 16, p, fo, nullptr, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_pack_weights(f, 16, 16, odd, fo, p, nullptr), BITLINEAR_ERR_ALIGN);
  EXPECT(bitlinear_pack_weights_b1(nullptr, 16, 16, p, fo, p, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_pack_weights_b3(f, 16, BITLINEAR_MAX_K + 1, p, fo, p, nullptr), BITLINEAR_ERR_SHAPE);

  // products
  EXPECT(bitlinear_gemv(q, f, 65, 16, p, f, 16, p, f32, nullptr, 0, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_gemv(q, f, 1, 16, p, f, 16, p, 9, nullptr, 0, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_gemv(q, f, 1, 16, odd, f, 16, p, f32, nullptr, 0, nullptr), BITLINEAR_ERR_ALIGN);
  EXPECT(bitlinear_gemv(nullptr, f, 1, 16, p, f, 16, p, f32, nullptr, 0, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_gemv(q, f, 0, 16, p, f, 16, p, f32, nullptr, 0, nullptr), BITLINEAR_OK);
  EXPECT(bitlinear_gemm(q, f, 1, 0, p, f, 16, p, f32, nullptr, 0, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_gemm(q, f, 1, 16, p, f, BITLINEAR_MAX_N + 1, p, f32, nullptr, 0, nullptr),
         BITLINEAR_ERR_SHAPE);
  {
    // a shape that needs a workspace, without one / with too short a one
    const int64_t need = bitlinear_gemm_workspace_bytes(32, 8192, 28672);
    CHECK(need > 0);
    EXPECT(bitlinear_gemm(q, f, 32, 28672, p, f, 8192, p, f32, nullptr, 0, nullptr), BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_gemm(q, f, 32, 28672, p, f, 8192, p, f32, p, (size_t)need - 1, nullptr), BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_gemm(q, f, 32, 28672, p, f, 8192, p, f32, odd, (size_t)need, nullptr), BITLINEAR_ERR_ALIGN);
  }
  EXPECT(bitlinear_gemv_b1(q, f, nullptr, 1, 16, p, f, 16, p, f32, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_gemv_b1(q, f, (const int32_t*)odd, 1, 16, p, f, 16, p, f32, nullptr), BITLINEAR_ERR_ALIGN);
  EXPECT(bitlinear_gemm_b1(q, f, rs, 1, 16, p, f, 0, p, f32, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_gemv_b3(q, f, rs, 65, 16, p, f, 16, p, f32, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_gemv_b3(q, f, nullptr, 1, 16, p, f, 16, p, f32, nullptr), BITLINEAR_ERR_ARG);

  // fused decode, multi, gated pair, glue
  EXPECT(bitlinear_forward_decode(p, 5, 1, 16, p, f, 16, p, f32, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_forward_decode(p, bf, 64, BITLINEAR_MAX_K, p, f, 16, p, f32, nullptr), BITLINEAR_ERR_UNSUPPORTED);
  EXPECT(bitlinear_forward_decode(odd, f32, 1, 16, p, f, 16, p, f32, nullptr), BITLINEAR_ERR_ALIGN);
  {
    const void* pk[5] = {p, p, p, p, p};
    const float* bt[5] = {f, f, f, f, f};
    int64_t ns[5] = {16, 16, 16, 16, 16};
    void* ys[5] = {p, p, p, p, p};
    EXPECT(bitlinear_gemv_multi(q, f, 1, 16, 0, pk, bt, ns, ys, f32, nullptr), BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_gemv_multi(q, f, 1, 16, BITLINEAR_MULTI_MAX + 1, pk, bt, ns, ys, f32, nullptr),
           BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_gemv_multi(q, f, 1, 16, 2, nullptr, bt, ns, ys, f32, nullptr), BITLINEAR_ERR_ARG);
    ns[1] = 0;
    EXPECT(bitlinear_gemv_multi(q, f, 1, 16, 2, pk, bt, ns, ys, f32, nullptr), BITLINEAR_ERR_SHAPE);
    ns[1] = 16;
    pk[1] = odd;
    EXPECT(bitlinear_forward_decode_multi(p, bf, 1, 16, 2, pk, bt, ns, ys, f32, nullptr), BITLINEAR_ERR_ALIGN);
  }
  EXPECT(bitlinear_gemv_glu(q, f, 1, 16, p, f, nullptr, f, 16, fo, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_forward_decode_glu(p, bf, 1, 16, p, f, p, f, 16, (float*)odd, nullptr), BITLINEAR_ERR_ALIGN);
  EXPECT(bitlinear_relu2_mul(f, f, -1, fo, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_relu2_mul(nullptr, f, 4, fo, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_relu2_mul(f, f, 0, fo, nullptr), BITLINEAR_OK);

  // products with the next BitLinear's quantization in the epilogue
  {
    const void* pk[2] = {p, p};
    const float* bt[2] = {f, f};
    int64_t ns[2] = {64, 64};
    void* ys[2] = {p, p};
    EXPECT(bitlinear_decode_rq(q, f, 1, 256, 1, 0, pk, bt, ns, ys, BITLINEAR_BF16, (int8_t*)p, fo, 0, p, 16, nullptr),
           BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_decode_rq(q, f, 1, 256, 1, 1, pk, bt, ns, ys, f32, (int8_t*)p, fo, 0, p, 16, nullptr),
           BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_decode_rq(q, f, 1, 256, 1, 0, pk, bt, ns, ys, f32, (int8_t*)p, fo, 7, p, 16, nullptr),
           BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_decode_rq(q, f, 1, 256, 1, 0, pk, bt, ns, ys, f32, (int8_t*)p, fo, 0, p, 4, nullptr),
           BITLINEAR_ERR_ARG);
    EXPECT(bitlinear_decode_rq(q, f, 1, 256, 1, 0, pk, bt, ns, ys, f32, (int8_t*)odd, fo, 0, p, 16, nullptr),
           BITLINEAR_ERR_ALIGN);
    ns[1] = 32;
    EXPECT(bitlinear_decode_rq(q, f, 1, 256, 2, 1, pk, bt, ns, ys, f32, (int8_t*)p, fo, 0, p, 16, nullptr),
           BITLINEAR_ERR_SHAPE);
    EXPECT(bitlinear_decode_rq(q, f, 0, 256, 2, 0, pk, bt, ns, ys, f32, (int8_t*)p, fo, 0, p, 16, nullptr),
           BITLINEAR_OK);
  }

  // training products
  EXPECT(bitlinear_train_forward(p, 1, 16, p, f, 0, fo, nullptr), BITLINEAR_ERR_SHAPE);
  EXPECT(bitlinear_train_backward_input(nullptr, 1, 16, p, f, 16, fo, nullptr), BITLINEAR_ERR_ARG);
  EXPECT(bitlinear_train_backward_weight(p, odd, 1, 16, 16, fo, nullptr), BITLINEAR_ERR_ALIGN);

  // the error string belongs to the calling thread
  EXPECT(bitlinear_gemv(q, f, 65, 16, p, f, 16, p, f32, nullptr, 0, nullptr), BITLINEAR_ERR_SHAPE);
  std::thread th([] { CHECK(bitlinear_last_error()[0] == '\0'); });
  th.join();
  CHECK(bitlinear_last_error()[0] != '\0');

  if (failures)
    fprintf(stderr, "%d check(s) failed\n", failures);
  else
    printf("ABI driver: all checks passed\n");
  return failures != 0;
}
