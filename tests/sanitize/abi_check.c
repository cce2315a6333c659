/* Argument validation and plan building of the C ABI (include/bitnet.h), run
 * under AddressSanitizer and UndefinedBehaviorSanitizer on the host.  No call
 * here reaches a kernel launch: each one fails its checks, is an empty no-op,
 * or only builds a plan image in host memory.  Plan buffers are allocated at
 * exactly the size the library asks for, so a write past the image is caught.
 * Prints "abi_check: N checks passed" and exits 0, or names each failed check. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bitnet.h"

static int g_checks, g_failed;

#define CHECK(expr)                                                        \
    do {                                                                   \
        ++g_checks;                                                        \
        if (!(expr)) {                                                     \
            ++g_failed;                                                    \
            fprintf(stderr, "abi_check:%d: failed: %s\n", __LINE__, #expr); \
        }                                                                  \
    } while (0)

/* never dereferenced: the calls below stop at their checks */
#define P(a) ((void *)(uintptr_t)(a))
static void *const p = P(4096);

static uint32_t hdr_word(const void *plan, int i) {
    uint32_t v;
    memcpy(&v, (const char *)plan + 4 * i, 4);
    return v;
}

static void status_strings(void) {
    for (int s = 0; s <= 5; ++s) CHECK(strncmp(bitnet_status_str(s), "BITNET_", 7) == 0);
    CHECK(bitnet_status_str(-1) != NULL && bitnet_status_str(99) != NULL);
    CHECK(bitnet_version() == 100);
    CHECK(bitnet_last_error() != NULL);
}

static void linear_checks(void) {
    CHECK(bitnet_linear(NULL, p, p, p, 1, 1, 64, p, NULL, NULL) == BITNET_ERR_NULL);
    CHECK(bitnet_linear(p, p, p, p, 1, 1, 6, p, NULL, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_linear(p, p, p, p, 1, 1, 0, p, NULL, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_linear(p, p, p, p, -1, 1, 64, p, NULL, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_linear(p, p, p, p, INT64_MAX, INT64_MAX, 64, p, NULL, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_linear(p, p, p, p, 1, 1, INT64_MAX - 3, p, NULL, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_linear(p, P(4097), p, p, 1, 1, 64, p, NULL, NULL) == BITNET_ERR_ALIGN);
    CHECK(bitnet_linear(NULL, NULL, NULL, NULL, 0, 5, 64, NULL, NULL, NULL) == BITNET_OK);
    CHECK(bitnet_linear_select(p, p, p, p, 1, 1, 64, p, NULL, -1, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_linear_select(p, p, p, p, 1, 1, 64, p, NULL, 1 << 30, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, NULL, p, 2, NULL, 0, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_linear_ex(p, p, p, p, 96, 1, 1, 128, NULL, p, BITNET_F32, NULL, 0, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_linear_ex(p, p, p, p, -64, 1, 1, 128, NULL, p, BITNET_F32, NULL, 0, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, P(4098), p, BITNET_F32, NULL, 0, NULL) == BITNET_ERR_ALIGN);
    CHECK(bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, NULL, P(4097), BITNET_BF16, NULL, 0, NULL) == BITNET_ERR_ALIGN);
}

static void pack_and_quant_checks(void) {
    CHECK(bitnet_pack_workspace_bytes(10, 64) == 80);
    CHECK(bitnet_pack_weights(NULL, 2, 64, 1e-5f, p, p, p, 16, NULL) == BITNET_ERR_NULL);
    CHECK(bitnet_pack_weights(p, 2, 62, 1e-5f, p, p, p, 16, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_pack_weights(p, 2, 64, 1e-5f, p, p, p, 8, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_pack_weights(p, 2, 64, 1e-5f, p, p, P(4100), 16, NULL) == BITNET_ERR_ALIGN);
    CHECK(bitnet_pack_weights_noalloc(p, (int64_t)BITNET_PACK_NOALLOC_MAX_ROWS + 1, 64, 1e-5f, p, p, NULL) ==
          BITNET_ERR_SHAPE);
    CHECK(bitnet_pack_weights_noalloc(NULL, 2, 64, 1e-5f, p, p, NULL) == BITNET_ERR_NULL);
    CHECK(bitnet_pack_weights_grouped(p, 2, 64, 0, 1e-5f, p, p, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_pack_weights_grouped(p, 2, 64, 48, 1e-5f, p, p, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_quant_act(NULL, 1, 64, p, p, NULL) == BITNET_ERR_NULL);
    CHECK(bitnet_quant_act(p, 1, 66, p, p, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_quant_act(P(4097), 1, 64, p, p, NULL) == BITNET_ERR_ALIGN);
    CHECK(bitnet_quant_act(NULL, 0, 64, NULL, NULL, NULL) == BITNET_OK);
    CHECK(bitnet_rmsnorm_quant_act(p, p, -1.0f, 1, 64, p, p, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_rmsnorm_quant_act(p, p, NAN, 1, 64, p, p, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_swiglu_quant_act(p, p, 1, 60, p, p, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_pack_weights_binary(p, 4, 48, p, p, p, 1 << 20, NULL) == BITNET_ERR_SHAPE);
    CHECK(bitnet_pack_weights_binary(p, 4, 64, p, p, p, 8, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_pack_bitplanes(NULL, 4, 64, p, NULL) == BITNET_ERR_NULL);
    CHECK(bitnet_linear_bits(p, p, p, 3, p, 1, 8, 128, p, NULL, 0, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_linear_bits(p, p, p, 1, p, 1, 8, 57344 + 128, p, NULL, 2, NULL) == BITNET_ERR_ARG);
}

/* a plan image in a buffer of exactly the size the library reports */
static void *plan_linear(const bitnet_linear_desc *d, int n, int *st) {
    const size_t nb = bitnet_grouped_plan_bytes(n, 1, d);
    void *buf = malloc(nb);
    *st = bitnet_grouped_plan_linear(d, n, buf, nb);
    if (*st == BITNET_OK) CHECK(bitnet_grouped_plan_linear(d, n, buf, nb - 1) == BITNET_ERR_ARG);
    return buf;
}

static void *plan_fused(const bitnet_fused_desc *d, int n, int *st) {
    const size_t nb = bitnet_grouped_plan_fused_bytes(n, d);
    void *buf = malloc(nb);
    *st = bitnet_grouped_plan_fused(d, n, buf, nb);
    return buf;
}

static void linear_plans(void) {
    /* many descriptors of mixed shapes: the image's descriptor and block tables */
    enum { ND = 97 };
    bitnet_linear_desc *d = calloc(ND, sizeof *d);
    for (int i = 0; i < ND; ++i) {
        d[i].q = p; d[i].s_x = p; d[i].packed = p; d[i].s_w = p; d[i].y = p;
        d[i].M = 1; d[i].N = 1 + 37 * i; d[i].K = 64 * (1 + i % 40);
    }
    int st;
    void *plan = plan_linear(d, ND, &st);
    CHECK(st == BITNET_OK);
    CHECK(hdr_word(plan, 0) != 0 && hdr_word(plan, 2) == ND && hdr_word(plan, 7) == 0);
    free(plan);
    for (int i = 0; i < ND; ++i) d[i].M = 1 + i % 16;      /* MFMA decode variant */
    plan = plan_linear(d, ND, &st);
    CHECK(st == BITNET_OK && hdr_word(plan, 7) == 1);
    free(plan);
    for (int i = 0; i < ND; ++i) d[i].w_group = (i % 3) ? 0 : 64;   /* group-wise, several tokens: MFMA decode */
    plan = plan_linear(d, ND, &st);
    CHECK(st == BITNET_OK && hdr_word(plan, 7) == 4);
    free(plan);
    for (int i = 0; i < ND; ++i) d[i].M = 1;                /* group-wise, one token each */
    plan = plan_linear(d, ND, &st);
    CHECK(st == BITNET_OK && hdr_word(plan, 7) == 2);
    free(plan);
    for (int i = 0; i < ND; ++i) d[i].M = 1 + i % 16;
    d[5].M = 17;
    plan = plan_linear(d, ND, &st);
    CHECK(st == BITNET_ERR_SHAPE);
    free(plan);
    d[5].M = 1;
    d[7].packed = P(4100);
    plan = plan_linear(d, ND, &st);
    CHECK(st == BITNET_ERR_ALIGN);
    free(plan);
    free(d);

    /* a linear plan is not a quant or fused plan; a zeroed buffer is not a plan */
    bitnet_linear_desc one = {.q = p, .s_x = p, .packed = p, .s_w = p, .y = p, .M = 1, .N = 100, .K = 2560};
    plan = plan_linear(&one, 1, &st);
    CHECK(st == BITNET_OK);
    CHECK(bitnet_quant_act_grouped(plan, p, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_linear_fused_grouped(plan, p, NULL) == BITNET_ERR_ARG);
    CHECK(bitnet_linear_grouped(plan, P(4100), NULL) == BITNET_ERR_ALIGN);
    void *junk = calloc(1, 128);
    CHECK(bitnet_linear_grouped(junk, p, NULL) == BITNET_ERR_ARG);
    free(junk);
    free(plan);

    bitnet_quant_desc qd[3] = {{.x = p, .q = p, .s_x = p, .M = 1, .K = 2560},
                               {.x = p, .q = p, .s_x = p, .M = 7, .K = 64},
                               {.x = p, .q = p, .s_x = p, .M = 2, .K = 6912}};
    const size_t qb = bitnet_grouped_plan_bytes(3, 0, qd);
    void *qplan = malloc(qb);
    CHECK(bitnet_grouped_plan_quant(qd, 3, qplan, qb) == BITNET_OK);
    CHECK(bitnet_grouped_plan_quant(qd, 3, qplan, qb - 1) == BITNET_ERR_ARG);
    CHECK(bitnet_linear_grouped(qplan, p, NULL) == BITNET_ERR_ARG);
    free(qplan);
}

static void fused_plans(void) {
    enum { ND = 31 };
    bitnet_fused_desc *d = calloc(ND, sizeof *d);
    for (int i = 0; i < ND; ++i) {
        d[i].x = p; d[i].packed = p; d[i].s_w = p; d[i].y = p;
        d[i].M = 1; d[i].N = 1 + 53 * i; d[i].K = 64 * (1 + i % 30);
        if (i % 4 == 1) { d[i].norm_gain = p; d[i].norm_eps = 1e-6f; }
        if (i % 4 == 2) { d[i].x = NULL; d[i].x_f32 = p; }
        if (i % 4 == 3) { d[i].packed_up = p; d[i].s_w_up = p; }
    }
    int st;
    void *plan = plan_fused(d, ND, &st);
    CHECK(st == BITNET_OK && hdr_word(plan, 1) == 3 && hdr_word(plan, 7) == 3);
    CHECK(bitnet_linear_grouped(plan, p, NULL) == BITNET_ERR_ARG);
    free(plan);
    d[3].acc = p;                        /* a gate / up pair takes no acc */
    plan = plan_fused(d, ND, &st);
    CHECK(st == BITNET_ERR_ARG);
    free(plan);
    d[3].acc = NULL;
    d[9].K = 52224 + 64;                 /* beyond one LDS segment */
    plan = plan_fused(d, ND, &st);
    CHECK(st == BITNET_ERR_SHAPE);
    free(plan);
    for (int i = 0; i < ND; ++i) {       /* bitplane plan: plain rows only */
        memset(&d[i], 0, sizeof d[i]);
        d[i].x = p; d[i].packed = p; d[i].s_w = p; d[i].y = p;
        d[i].M = 1; d[i].N = 1 + 53 * i; d[i].K = 64 * (1 + i % 30);
        d[i].weight_fmt = BITNET_FMT_BITPLANES;
    }
    plan = plan_fused(d, ND, &st);
    CHECK(st == BITNET_OK && hdr_word(plan, 7) == 4);
    free(plan);
    d[4].weight_fmt = 0;
    plan = plan_fused(d, ND, &st);
    CHECK(st == BITNET_ERR_ARG);
    free(plan);
    free(d);
}

int main(void) {
    status_strings();
    linear_checks();
    pack_and_quant_checks();
    linear_plans();
    fused_plans();
    if (g_failed) {
        fprintf(stderr, "abi_check: %d of %d checks failed\n", g_failed, g_checks);
        return 1;
    }
    printf("abi_check: %d checks passed\n", g_checks);
    return 0;
}
