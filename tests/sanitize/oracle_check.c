/* Every function of the CPU oracle (oracle/bitnet_oracle.c) on small inputs,
 * run under AddressSanitizer and UndefinedBehaviorSanitizer.  Buffers are
 * allocated at exactly the sizes the functions are documented to touch, so a
 * read or write past them is caught.  Results are checked against brute-force
 * sums written here (the product over unpacked codes, the dot product of the
 * +/-1 or sign / mask weights), which also ties the encodings together.
 * Prints "oracle_check: N checks passed" and exits 0, or names each failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_set_threads(int n);
float oracle_weight_scale(const float *w, int64_t N, int64_t K, double *rowsum);
void oracle_pack(const float *w, int64_t N, int64_t K, float eps, float s_w, uint8_t *packed);
void oracle_pack_grouped(const float *w, int64_t N, int64_t K, int64_t G, float eps, float *s_w, uint8_t *packed);
void oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *t);
void oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s_x);
void oracle_quant_act_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *s_x);
void oracle_rmsnorm_quant(const uint16_t *x, const float *g, float eps, int64_t M, int64_t K, int8_t *q,
                          float *s_x);
void oracle_swiglu_quant(const float *g, const float *u, int64_t M, int64_t K, float *a, int8_t *q, float *s_x);
void oracle_linear(const int8_t *q, const float *s_x, const uint8_t *packed, float s_w, int64_t M, int64_t N,
                   int64_t K, int32_t *acc, float *y);
void oracle_linear_bias(const int8_t *q, const float *s_x, const uint8_t *packed, float s_w, const float *bias,
                        int64_t M, int64_t N, int64_t K, int32_t *acc, float *y);
void oracle_linear_grouped(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w, int64_t G,
                           const float *bias, int64_t M, int64_t N, int64_t K, int32_t *acc, float *y);
void oracle_pack_binary(const float *w, int64_t N, int64_t K, uint8_t *bits);
void oracle_linear_binary(const int8_t *q, const float *s_x, const uint8_t *bits, float s_w, int64_t M, int64_t N,
                          int64_t K, int32_t *acc, float *y);
void oracle_pack_bitplanes(const uint8_t *packed, int64_t N, int64_t K, uint8_t *planes);
void oracle_linear_bitplanes(const int8_t *q, const float *s_x, const uint8_t *planes, float s_w, int64_t M,
                             int64_t N, int64_t K, int32_t *acc, float *y);
void oracle_to_bf16(const float *y, int64_t n, uint16_t *out);

static int g_checks, g_failed;

#define CHECK(expr)                                                           \
    do {                                                                      \
        ++g_checks;                                                           \
        if (!(expr)) {                                                        \
            ++g_failed;                                                       \
            fprintf(stderr, "oracle_check:%d: failed: %s\n", __LINE__, #expr); \
        }                                                                     \
    } while (0)

static uint64_t g_state = 0x243F6A8885A308D3ull;
static double uniform(void) {   /* xorshift64*, [-1, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

static uint16_t bf16_bits(float f) {   /* truncation: any bf16 value will do as input */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t n) {
    void *r = malloc(n ? n : 1);
    if (!r) abort();
    return r;
}

/* one shape: M tokens, N rows, K weights per row (K % 32 == 0 for the bit formats) */
static void run_shape(int64_t M, int64_t N, int64_t K, int bits_formats) {
    float *w = xmalloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < N * K; ++i) w[i] = (float)(0.05 * uniform());
    if (N > 1) for (int64_t k = 0; k < K; ++k) w[K + k] = 0.0f;   /* an all-zero row */
    double *rowsum = xmalloc(sizeof(double) * N);
    const float s_w = oracle_weight_scale(w, N, K, rowsum);
    double ref = 0.0;
    for (int64_t i = 0; i < N * K; ++i) ref += fabs((double)w[i]);
    if (N > 0) CHECK(fabs((double)s_w - ref / (double)(N * K)) <= 1e-6 * ref / (double)(N * K) + 1e-30);

    uint8_t *packed = xmalloc((size_t)(N * K / 4));
    oracle_pack(w, N, K, 1e-5f, s_w, packed);
    int8_t *t = xmalloc((size_t)(N * K));
    oracle_unpack(packed, N, K, t);
    int ternary = 1;
    for (int64_t i = 0; i < N * K; ++i) ternary &= (t[i] >= -1 && t[i] <= 1);
    CHECK(ternary);
    if (N > 1) {
        int zero = 1;
        for (int64_t k = 0; k < K; ++k) zero &= (t[K + k] == 0);
        CHECK(zero);
    }

    const int64_t G = K >= 8 && K % 8 == 0 ? K / 2 : K;
    float *s_wg = xmalloc(sizeof(float) * N * (K / G));
    uint8_t *packed_g = xmalloc((size_t)(N * K / 4));
    oracle_pack_grouped(w, N, K, G, 1e-5f, s_wg, packed_g);

    uint16_t *x = xmalloc(sizeof(uint16_t) * M * K);
    float *xf = xmalloc(sizeof(float) * M * K);
    float *gain = xmalloc(sizeof(float) * K);
    for (int64_t i = 0; i < M * K; ++i) {
        xf[i] = (float)(3.0 * uniform());
        x[i] = bf16_bits(xf[i]);
    }
    for (int64_t k = 0; k < K; ++k) gain[k] = (float)(1.0 + 0.5 * uniform());
    if (M > 1) for (int64_t k = 0; k < K; ++k) { x[K + k] = 0; xf[K + k] = 0.0f; }   /* an all-zero row */
    int8_t *q = xmalloc((size_t)(M * K));
    float *s_x = xmalloc(sizeof(float) * M);
    oracle_quant_act_f32(xf, M, K, q, s_x);
    oracle_rmsnorm_quant(x, gain, 1e-6f, M, K, q, s_x);
    float *a = xmalloc(sizeof(float) * M * K);
    oracle_swiglu_quant(xf, xf, M, K, a, q, s_x);
    oracle_quant_act(x, M, K, q, s_x);
    int in_range = 1;
    for (int64_t i = 0; i < M * K; ++i) in_range &= (q[i] >= -127 && q[i] <= 127);
    CHECK(in_range);

    int32_t *acc = xmalloc(sizeof(int32_t) * M * N), *acc2 = xmalloc(sizeof(int32_t) * M * N);
    float *y = xmalloc(sizeof(float) * M * N);
    float *bias = xmalloc(sizeof(float) * N);
    for (int64_t n = 0; n < N; ++n) bias[n] = (float)uniform();
    oracle_linear(q, s_x, packed, s_w, M, N, K, acc, y);
    int exact = 1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)q[m * K + k] * t[n * K + k];
            exact &= (s == acc[m * N + n]) && isfinite(y[m * N + n]);
        }
    CHECK(exact);
    oracle_linear_bias(q, s_x, packed, s_w, bias, M, N, K, acc2, y);
    CHECK(memcmp(acc, acc2, sizeof(int32_t) * M * N) == 0);
    oracle_linear_grouped(q, s_x, packed_g, s_wg, G, bias, M, N, K, acc2, y);
    oracle_linear_grouped(q, s_x, packed_g, s_wg, G, NULL, M, N, K, acc2, y);

    uint16_t *yb = xmalloc(sizeof(uint16_t) * M * N);
    oracle_to_bf16(y, M * N, yb);

    if (bits_formats) {
        uint8_t *bits = xmalloc((size_t)(N * K / 8));
        oracle_pack_binary(w, N, K, bits);
        oracle_linear_binary(q, s_x, bits, s_w, M, N, K, acc2, y);
        int ok = 1;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                int64_t s = 0;
                for (int64_t k = 0; k < K; ++k) s += (int64_t)q[m * K + k] * (w[n * K + k] >= 0.0f ? 1 : -1);
                ok &= (s == acc2[m * N + n]);
            }
        CHECK(ok);
        uint8_t *planes = xmalloc((size_t)(N * (K / 32) * 8));
        oracle_pack_bitplanes(packed, N, K, planes);
        oracle_linear_bitplanes(q, s_x, planes, s_w, M, N, K, acc2, y);
        CHECK(memcmp(acc, acc2, sizeof(int32_t) * M * N) == 0);
        free(bits);
        free(planes);
    }
    free(w); free(rowsum); free(packed); free(t); free(s_wg); free(packed_g); free(x); free(xf); free(gain);
    free(q); free(s_x); free(a); free(acc); free(acc2); free(y); free(bias); free(yb);
}

int main(void) {
    oracle_set_threads(2);
    run_shape(1, 1, 4, 0);
    run_shape(3, 5, 36, 0);
    run_shape(2, 7, 96, 1);
    run_shape(5, 33, 320, 1);
    run_shape(0, 3, 64, 1);     /* no tokens */
    run_shape(2, 0, 64, 1);     /* no rows */
    if (g_failed) {
        fprintf(stderr, "oracle_check: %d of %d checks failed\n", g_failed, g_checks);
        return 1;
    }
    printf("oracle_check: %d checks passed\n", g_checks);
    return 0;
}
