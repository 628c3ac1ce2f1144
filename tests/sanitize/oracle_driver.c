/*
 * Drives every function of the CPU oracle (oracle/bitlinear_oracle.c) on
 * small and edge-case shapes, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  It checks the round trips and invariants that
 * need no second implementation; the sanitizers check every access and every
 * integer operation.  Exit status 0 means every check passed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_absmean(const float *w, int64_t count);
void oracle_ternarize(const float *w, int64_t count, float beta, int8_t *t);
void oracle_quant_act_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *ds, int32_t *rowsum);
void oracle_quant_act_bf16(const uint16_t *xb, int64_t M, int64_t K, int8_t *q, float *ds, int32_t *rowsum);
void oracle_matmul_i32(const int8_t *q, const int8_t *t, int64_t M, int64_t N, int64_t K, int32_t *acc,
                       int threads);
void oracle_matmul_i32_pairs(const int8_t *q, const int8_t *t, int64_t K, const int64_t *ms, const int64_t *ns,
                             int64_t count, int32_t *out);
void oracle_dequant_f32(const int32_t *acc, const float *ds, float beta, int64_t M, int64_t N, float *y);
void oracle_f32_to_bf16(const float *y, int64_t count, uint16_t *out);
int64_t oracle_t2_bytes(int64_t N, int64_t K);
void oracle_pack_t2(const int8_t *t, int64_t N, int64_t K, uint8_t *packed);
int64_t oracle_unpack_t2(const uint8_t *packed, int64_t N, int64_t K, int8_t *t);
int64_t oracle_b1_bytes(int64_t N, int64_t K);
void oracle_binarize(const float *w, int64_t count, int8_t *t);
void oracle_pack_b1(const int8_t *t, int64_t N, int64_t K, uint8_t *packed);
void oracle_unpack_b1(const uint8_t *packed, int64_t N, int64_t K, int8_t *t);
int64_t oracle_b3_bytes(int64_t N, int64_t K);
void oracle_pack_b3(const int8_t *t, int64_t N, int64_t K, uint8_t *packed);
void oracle_unpack_b3(const uint8_t *packed, int64_t N, int64_t K, int8_t *t);
void oracle_relu2_mul(const float *g, const float *u, int64_t count, float *h);
void oracle_add_f32(float *x, const float *r, int64_t count);
void oracle_rmsnorm_f32(const float *x, int64_t M, int64_t K, float *xn);
void oracle_train_forward(const uint16_t *xb, int64_t M, int64_t K, const int8_t *t, float beta, int64_t N,
                          float *y, int threads);
void oracle_train_dx(const uint16_t *dyb, int64_t M, int64_t N, const int8_t *t, float beta, int64_t K,
                     float *dx, int threads);
void oracle_train_dw(const uint16_t *dyb, const uint16_t *xb, int64_t M, int64_t N, int64_t K, float *dw,
                     int threads);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}
/* uniform in [-1, 1) with a few exact zeros */
static float next_f(void)
{
    uint32_t u = next_u32();
    if ((u & 31u) == 0)
        return 0.0f;
    return (float)((int32_t)(u >> 8) - (1 << 23)) / (float)(1 << 23);
}

static int failures = 0;
#define CHECK(cond, ...)                         \
    do {                                         \
        if (!(cond)) {                           \
            fprintf(stderr, __VA_ARGS__);        \
            fprintf(stderr, "\n");               \
            ++failures;                          \
        }                                        \
    } while (0)

/* Exact-size heap buffers, so an access one past the end is reported. */
#define NEW(type, n) ((type *)malloc(((size_t)(n) > 0 ? (size_t)(n) : 1) * sizeof(type)))

static void run_shape(int64_t M, int64_t N, int64_t K)
{
    float *w = NEW(float, N * K), *x = NEW(float, M * K);
    uint16_t *xb = NEW(uint16_t, M * K), *dyb = NEW(uint16_t, M * N);
    for (int64_t i = 0; i < N * K; ++i)
        w[i] = 0.02f * next_f();
    for (int64_t i = 0; i < M * K; ++i)
        x[i] = 4.0f * next_f();
    if (M > 1)
        memset(x + K, 0, (size_t)K * sizeof(float)); /* an all-zero token row */
    oracle_f32_to_bf16(x, M * K, xb);
    for (int64_t i = 0; i < M * N; ++i) {
        float v = next_f();
        oracle_f32_to_bf16(&v, 1, dyb + i);
    }

    float beta = oracle_absmean(w, N * K);
    int8_t *t = NEW(int8_t, N * K), *t2 = NEW(int8_t, N * K);
    oracle_ternarize(w, N * K, beta, t);
    for (int64_t i = 0; i < N * K; ++i)
        CHECK(t[i] >= -1 && t[i] <= 1, "ternary code %d out of range", t[i]);

    int8_t *q = NEW(int8_t, M * K);
    float *ds = NEW(float, M);
    int32_t *rs = NEW(int32_t, M);
    oracle_quant_act_f32(x, M, K, q, ds, rs);
    oracle_quant_act_bf16(xb, M, K, q, ds, rs);
    for (int64_t i = 0; i < M * K; ++i)
        CHECK(q[i] >= -127 && q[i] <= 127, "int8 code %d out of range", q[i]);

    int32_t *acc = NEW(int32_t, M * N), *acc2 = NEW(int32_t, M * N);
    oracle_matmul_i32(q, t, M, N, K, acc, 1);
    oracle_matmul_i32(q, t, M, N, K, acc2, 3);
    CHECK(memcmp(acc, acc2, (size_t)(M * N) * sizeof(int32_t)) == 0, "threaded product differs");
    int64_t ms[2] = {0, M - 1}, ns[2] = {N - 1, 0};
    int32_t pr[2];
    oracle_matmul_i32_pairs(q, t, K, ms, ns, 2, pr);
    CHECK(pr[0] == acc[N - 1] && pr[1] == acc[(M - 1) * N], "pair products differ");

    float *y = NEW(float, M * N);
    uint16_t *yb = NEW(uint16_t, M * N);
    oracle_dequant_f32(acc, ds, beta, M, N, y);
    oracle_f32_to_bf16(y, M * N, yb);

    uint8_t *p2 = NEW(uint8_t, oracle_t2_bytes(N, K));
    oracle_pack_t2(t, N, K, p2);
    CHECK(oracle_unpack_t2(p2, N, K, t2) == 0, "invalid 2-bit codes");
    CHECK(memcmp(t, t2, (size_t)(N * K)) == 0, "2-bit round trip differs");

    uint8_t *p3 = NEW(uint8_t, oracle_b3_bytes(N, K));
    oracle_pack_b3(t, N, K, p3);
    oracle_unpack_b3(p3, N, K, t2);
    CHECK(memcmp(t, t2, (size_t)(N * K)) == 0, "base-3 round trip differs");

    int8_t *tb = NEW(int8_t, N * K);
    oracle_binarize(w, N * K, tb);
    uint8_t *p1 = NEW(uint8_t, oracle_b1_bytes(N, K));
    oracle_pack_b1(tb, N, K, p1);
    oracle_unpack_b1(p1, N, K, t2);
    CHECK(memcmp(tb, t2, (size_t)(N * K)) == 0, "1-bit round trip differs");

    float *g = NEW(float, M * N), *h = NEW(float, M * N), *xn = NEW(float, M * K);
    for (int64_t i = 0; i < M * N; ++i)
        g[i] = next_f();
    oracle_relu2_mul(g, y, M * N, h);
    oracle_add_f32(h, y, M * N);
    oracle_rmsnorm_f32(x, M, K, xn);

    float *ty = NEW(float, M * N), *tdx = NEW(float, M * K), *tdw = NEW(float, N * K);
    oracle_train_forward(xb, M, K, t, beta, N, ty, 2);
    oracle_train_dx(dyb, M, N, t, beta, K, tdx, 2);
    oracle_train_dw(dyb, xb, M, N, K, tdw, 2);

    free(w), free(x), free(xb), free(dyb), free(t), free(t2), free(q), free(ds), free(rs);
    free(acc), free(acc2), free(y), free(yb), free(p2), free(p3), free(tb), free(p1);
    free(g), free(h), free(xn), free(ty), free(tdx), free(tdw);
}

int main(void)
{
    static const int64_t shapes[][3] = {{1, 1, 1},   {1, 16, 256}, {3, 17, 257}, {2, 35, 700},
                                        {4, 5, 3},   {1, 1, 4097}, {2, 16, 512}, {3, 33, 1000},
                                        {1, 64, 64}, {5, 3, 321}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        run_shape(shapes[i][0], shapes[i][1], shapes[i][2]);
    /* all-zero weights: beta = 0, every code 0 */
    float z[12] = {0};
    int8_t tz[12];
    float bz = oracle_absmean(z, 12);
    oracle_ternarize(z, 12, bz, tz);
    for (int i = 0; i < 12; ++i)
        CHECK(tz[i] == 0, "zero weight gave code %d", tz[i]);
    if (failures)
        fprintf(stderr, "%d check(s) failed\n", failures);
    else
        printf("oracle driver: all checks passed\n");
    return failures != 0;
}
