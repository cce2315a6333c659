// C ABI of the library: argument checks on the host, then dispatch to the gfx950
// kernels.  Checks never touch the GPU, so a failed check enqueues nothing.
#define BITNET_BUILD 1
#include "bitnet.h"
#include "bitnet_probe.h"

#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "internal.h"

using namespace bitnet;

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // kernels index rows and columns with int32
constexpr int64_t kGemvMaxM = 16;

int fail(int status, const char *msg) {
    g_last_error = msg;
    return status;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return BITNET_OK;
    g_last_error = hipGetErrorString(e);
    return BITNET_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_dims(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K <= 0 || K % 4 != 0) return fail(BITNET_ERR_SHAPE, "bad M/N/K");
    if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return fail(BITNET_ERR_SHAPE, "dimension too large");
    if (M * K >= ((int64_t)1 << 40) || N * K >= ((int64_t)1 << 42) || M * N >= ((int64_t)1 << 40))
        return fail(BITNET_ERR_SHAPE, "problem too large");
    return BITNET_OK;
}

int check_linear(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                 int64_t M, int64_t N, int64_t K, const float *y, const int32_t *acc) {
    int st = check_dims(M, N, K);
    if (st) return st;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!q || !s_x || !packed || !s_w || !y) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(s_x, 4) || !aligned(s_w, 4) || !aligned(y, 4) || (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "s_x, s_w, y and acc must be 4-byte aligned");
    return BITNET_OK;
}

bool linear_fast(const int8_t *q, const uint8_t *packed, int64_t K) {
    return K % 64 == 0 && aligned(q, 16) && aligned(packed, 16);
}

}  // namespace

extern "C" {

BITNET_API const char *bitnet_status_str(int s) {
    switch (s) {
        case BITNET_OK: return "BITNET_OK";
        case BITNET_ERR_NULL: return "BITNET_ERR_NULL: a required pointer is NULL";
        case BITNET_ERR_SHAPE: return "BITNET_ERR_SHAPE: invalid M, N, K or count";
        case BITNET_ERR_ALIGN: return "BITNET_ERR_ALIGN: misaligned pointer";
        case BITNET_ERR_HIP: return "BITNET_ERR_HIP: the HIP runtime reported an error";
        case BITNET_ERR_ARG: return "BITNET_ERR_ARG: invalid argument";
        default: return "unknown bitnet status";
    }
}

BITNET_API const char *bitnet_last_error(void) { return g_last_error.c_str(); }

BITNET_API int bitnet_version(void) { return 100; }

// ----------------------------------------------------------------- probes

BITNET_API int bitnet_probe_stream_read(const void *buf, size_t bytes, int64_t blocks, uint32_t key,
                                        uint32_t *sink, void *stream) {
    if (!buf || !sink) return fail(BITNET_ERR_NULL, "null pointer");
    if (bytes == 0 || bytes % 16 != 0 || bytes >= ((size_t)1 << 40) || blocks < 1 || blocks > 65536)
        return fail(BITNET_ERR_SHAPE, "bytes must be a nonzero multiple of 16 below 2^40, blocks 1 .. 65536");
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(BITNET_ERR_ALIGN, "buf 16-byte, sink 4-byte aligned");
    return hip_status(launch_probe_stream_read(buf, (int64_t)bytes, blocks, key, sink, (hipStream_t)stream));
}

BITNET_API int bitnet_probe_mfma_i8(int64_t blocks, int64_t iters, uint32_t key, uint32_t *sink, void *stream) {
    if (!sink) return fail(BITNET_ERR_NULL, "null pointer");
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > ((int64_t)1 << 24))
        return fail(BITNET_ERR_SHAPE, "blocks 1 .. 65536, iters 1 .. 2^24");
    if (!aligned(sink, 4)) return fail(BITNET_ERR_ALIGN, "sink 4-byte aligned");
    return hip_status(launch_probe_mfma_i8(blocks, iters, key, sink, (hipStream_t)stream));
}

BITNET_API double bitnet_probe_mfma_i8_ops(int64_t blocks, int64_t iters) { return probe_mfma_i8_ops(blocks, iters); }

BITNET_API size_t bitnet_pack_workspace_bytes(int64_t N, int64_t K) {
    (void)K;
    return N > 0 ? (size_t)N * sizeof(double) : 0;
}

BITNET_API int bitnet_pack_weights(const float *w, int64_t N, int64_t K, float eps, uint8_t *packed,
                                   float *s_w, void *workspace, size_t workspace_bytes, void *stream) {
    int st = check_dims(0, N, K);
    if (st) return st;
    if (!s_w) return fail(BITNET_ERR_NULL, "s_w is NULL");
    if (N > 0 && (!w || !packed || !workspace)) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(s_w, 4) || (w && !aligned(w, 4)) || (workspace && !aligned(workspace, 8)))
        return fail(BITNET_ERR_ALIGN, "w, s_w must be 4-byte and workspace 8-byte aligned");
    if (workspace_bytes < bitnet_pack_workspace_bytes(N, K))
        return fail(BITNET_ERR_ARG, "workspace too small");
    return hip_status(launch_pack(w, N, K, eps, packed, s_w, (double *)workspace, (hipStream_t)stream));
}

BITNET_API int bitnet_pack_weights_noalloc(const float *w, int64_t N, int64_t K, float eps, uint8_t *packed,
                                           float *s_w, void *stream) {
    static_assert(BITNET_PACK_NOALLOC_MAX_ROWS == kPackScratchRows, "header and library disagree");
    int st = check_dims(0, N, K);
    if (st) return st;
    if (N > BITNET_PACK_NOALLOC_MAX_ROWS) return fail(BITNET_ERR_SHAPE, "N exceeds the library's scratch rows");
    if (!s_w) return fail(BITNET_ERR_NULL, "s_w is NULL");
    if (N > 0 && (!w || !packed)) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(s_w, 4) || (w && !aligned(w, 4))) return fail(BITNET_ERR_ALIGN, "w and s_w must be 4-byte aligned");
    double *rowsum = nullptr;
    hipError_t e = pack_scratch(&rowsum);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_pack(w, N, K, eps, packed, s_w, rowsum, (hipStream_t)stream));
}

BITNET_API int bitnet_pack_weights_binary(const float *w, int64_t N, int64_t K, uint8_t *bits, float *s_w,
                                          void *workspace, size_t workspace_bytes, void *stream) {
    int st = check_dims(0, N, K);
    if (st) return st;
    if (K % 32 != 0) return fail(BITNET_ERR_SHAPE, "K must be a multiple of 32");
    if (!s_w) return fail(BITNET_ERR_NULL, "s_w is NULL");
    if (N > 0 && (!w || !bits || !workspace)) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(s_w, 4) || (w && !aligned(w, 16)) || (bits && !aligned(bits, 4)) ||
        (workspace && !aligned(workspace, 8)))
        return fail(BITNET_ERR_ALIGN, "w must be 16-byte, bits and s_w 4-byte, workspace 8-byte aligned");
    if (workspace_bytes < bitnet_pack_workspace_bytes(N, K)) return fail(BITNET_ERR_ARG, "workspace too small");
    hipError_t e = launch_weight_scale(w, N, K, s_w, (double *)workspace, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_pack_binary(w, N, K, bits, (hipStream_t)stream);
    return hip_status(e);
}

BITNET_API int bitnet_pack_bitplanes(const uint8_t *packed, int64_t N, int64_t K, uint8_t *planes, void *stream) {
    int st = check_dims(0, N, K);
    if (st) return st;
    if (K % 32 != 0) return fail(BITNET_ERR_SHAPE, "K must be a multiple of 32");
    if (N == 0) return BITNET_OK;
    if (!packed || !planes) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(packed, 8) || !aligned(planes, 8)) return fail(BITNET_ERR_ALIGN, "packed and planes must be 8-byte aligned");
    return hip_status(launch_pack_bitplanes(packed, N, K, planes, (hipStream_t)stream));
}

BITNET_API int bitnet_linear_bits(const int8_t *q, const float *s_x, const uint8_t *wbits, int fmt, const float *s_w,
                                  int64_t M, int64_t N, int64_t K, float *y, int32_t *acc, int kernel, void *stream) {
    if (fmt != BITNET_FMT_BINARY && fmt != BITNET_FMT_BITPLANES) return fail(BITNET_ERR_ARG, "unknown weight format");
    if (kernel < 0 || kernel > 4) return fail(BITNET_ERR_ARG, "unknown kernel id");
    int st = check_dims(M, N, K);
    if (st) return st;
    if (K % 32 != 0) return fail(BITNET_ERR_SHAPE, "K must be a multiple of 32");
    if (M == 0 || N == 0) return BITNET_OK;
    if (!q || !s_x || !wbits || !s_w || !y) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(s_x, 4) || !aligned(s_w, 4) || !aligned(y, 4) || (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "s_x, s_w, y and acc must be 4-byte aligned");
    if (kernel == 2 && !bits_fast_ok(fmt, M, K, q, wbits))
        return fail(BITNET_ERR_ARG, "the bit-serial GEMV needs M == 1, K % 128 (binary) or % 64 (bitplanes), "
                                    "K within its LDS limit, 16-byte aligned q and weights");
    if (kernel == 3 && (!bits_mt_ok(fmt, K, q, wbits) || M > 65535))
        return fail(BITNET_ERR_ARG, "the multi-token bit-serial kernel needs K % 128 (binary) or % 64 (bitplanes), "
                                    "one token's planes within 64 KiB of LDS, M <= 65535, 16-byte aligned q and weights");
    if (kernel == 4 && !bits_mfma_ok(fmt, M, K, q, wbits))
        return fail(BITNET_ERR_ARG, "the matrix-core kernel needs K % 64 == 0, at most 65535 tiles of 16 tokens, "
                                    "16-byte aligned q and weights");
    return hip_status(launch_linear_bits(q, s_x, wbits, fmt, s_w, M, N, K, y, acc, kernel, (hipStream_t)stream));
}

BITNET_API int bitnet_pack_weights_grouped(const float *w, int64_t N, int64_t K, int64_t group, float eps,
                                           uint8_t *packed, float *s_w, void *stream) {
    int st = check_dims(0, N, K);
    if (st) return st;
    if (group <= 0 || K % group != 0 || group % 4 != 0)
        return fail(BITNET_ERR_SHAPE, "group must be a positive multiple of 4 dividing K");
    if (N == 0) return BITNET_OK;
    if (!w || !packed || !s_w) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(w, 4) || !aligned(s_w, 4)) return fail(BITNET_ERR_ALIGN, "w and s_w must be 4-byte aligned");
    return hip_status(launch_pack_grouped(w, N, K, group, eps, packed, s_w, (hipStream_t)stream));
}

BITNET_API int bitnet_quant_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s_x,
                                void *stream) {
    int st = check_dims(M, 1, K);
    if (st) return st;
    if (M == 0) return BITNET_OK;
    if (!x || !q || !s_x) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(x, 2) || !aligned(s_x, 4)) return fail(BITNET_ERR_ALIGN, "x must be 2-byte, s_x 4-byte aligned");
    return hip_status(launch_quant_act(x, M, K, q, s_x, (hipStream_t)stream));
}

BITNET_API int bitnet_rmsnorm_quant_act(const uint16_t *x, const float *gain, float eps, int64_t M, int64_t K,
                                        int8_t *q, float *s_x, void *stream) {
    int st = check_dims(M, 1, K);
    if (st) return st;
    if (M == 0) return BITNET_OK;
    if (!x || !gain || !q || !s_x) return fail(BITNET_ERR_NULL, "null pointer");
    if (K % 8 != 0) return fail(BITNET_ERR_SHAPE, "K must be a multiple of 8");
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(gain, 16) || !aligned(s_x, 4) || (K * 2) % 16 != 0)
        return fail(BITNET_ERR_ALIGN, "x, q and gain must be 16-byte aligned (rows too), s_x 4-byte");
    if (!(eps >= 0.0f) || eps > 3.4e38f) return fail(BITNET_ERR_ARG, "eps must be finite and >= 0");
    return hip_status(launch_rmsnorm_quant(x, gain, eps, M, K, q, s_x, (hipStream_t)stream));
}

BITNET_API int bitnet_swiglu_quant_act(const float *gate, const float *up, int64_t M, int64_t K, int8_t *q,
                                       float *s_x, void *stream) {
    int st = check_dims(M, 1, K);
    if (st) return st;
    if (M == 0) return BITNET_OK;
    if (!gate || !up || !q || !s_x) return fail(BITNET_ERR_NULL, "null pointer");
    if (K % 8 != 0) return fail(BITNET_ERR_SHAPE, "K must be a multiple of 8");
    if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(q, 16) || !aligned(s_x, 4))
        return fail(BITNET_ERR_ALIGN, "gate, up and q must be 16-byte aligned, s_x 4-byte");
    return hip_status(launch_swiglu_quant(gate, up, M, K, q, s_x, (hipStream_t)stream));
}

BITNET_API int bitnet_linear_ex(const int8_t *q, const float *s_x, const uint8_t *packed,
                                const float *s_w, int64_t w_group, int64_t M, int64_t N, int64_t K,
                                const float *bias, void *y, int y_dtype, int32_t *acc, int kernel,
                                void *stream) {
    const bool forced_tile = kernel >= 16 && kernel < 16 + gemm_config_count();
    if ((kernel < 0 || kernel > 4) && !forced_tile) return fail(BITNET_ERR_ARG, "unknown kernel id");
    if (y_dtype != BITNET_F32 && y_dtype != BITNET_BF16) return fail(BITNET_ERR_ARG, "unknown output dtype");
    int st = check_dims(M, N, K);
    if (st) return st;
    if (w_group < 0 || (w_group > 0 && (K % w_group != 0 || w_group % 4 != 0)))
        return fail(BITNET_ERR_SHAPE, "w_group must be 0 or a multiple of 4 dividing K");
    // group-wise scales below the row length: the decode GEMV, the general kernel, or
    // the pipelined GEMM (kernel 2, tiles 21 / 22) without acc
    const bool groups = w_group > 0 && w_group < K;
    const bool pipe_tile = kernel == 16 + 5 || kernel == 16 + 6;
    if (groups && kernel != 0 && kernel != 1 && kernel != 3) {
        if ((kernel != 2 && !pipe_tile) || acc || !gemm_pipe_groups_ok(M, N, K, w_group))
            return fail(BITNET_ERR_ARG, "group-wise weight scales need kernel 0, 1 or 3, or the GEMM (2, 21, 22) "
                                        "with no acc, K % 128 == 0 and w_group 64 or a multiple of 128");
    }
    if (M == 0 || N == 0) return BITNET_OK;
    if (!q || !s_x || !packed || !s_w || !y) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(s_x, 4) || !aligned(s_w, 4) || (acc && !aligned(acc, 4)) || (bias && !aligned(bias, 4)))
        return fail(BITNET_ERR_ALIGN, "s_x, s_w, bias and acc must be 4-byte aligned");
    if (!aligned(y, y_dtype == BITNET_BF16 ? 2 : 4))
        return fail(BITNET_ERR_ALIGN, "y must be aligned to its element size");
    const OutSpec out{y, bias, y_dtype == BITNET_BF16 ? 1 : 0, (int)w_group};
    hipStream_t s = (hipStream_t)stream;
    const bool fast = linear_fast(q, packed, K) && (!groups || w_group % 64 == 0);
    if (kernel == 3 || (kernel == 0 && !fast))
        return hip_status(launch_linear_generic(q, s_x, packed, s_w, M, N, K, out, acc, s));
    if (!fast)
        return fail(BITNET_ERR_ALIGN, "kernel needs K % 64 == 0, 16-byte aligned q/packed (and w_group % 64 == 0)");
    // one token: the GEMV, except below 32 MB of packed weights, where the MFMA decode
    // kernel's shorter critical path wins (0.4 .. 17 MB: 4.3 .. 6.2 us against 5.6 ..
    // 7.3 us; from 58.7 MB on the GEMV streams faster); up to 16 tokens: the MFMA decode
    // kernel; beyond, whichever of the MFMA decode kernel (one 16-token tile per pass
    // over the weights) and the GEMM (few tiles, each walking all of K, when M and N are
    // small) is estimated faster; group-wise scales: the GEMV
    if (kernel == 0) {
        const bool small = N * (K / 4) < ((int64_t)32 << 20);
        if (groups) kernel = (M > kGemvMaxM && !acc && gemm_pipe_groups_ok(M, N, K, w_group)) ? 2 : 1;
        else if (M == 1 && !small) kernel = 1;
        else if (M <= kGemvMaxM || skinny_estimate_us(M, N, K) <= gemm_estimate_us(M, N, K)) kernel = 4;
        else kernel = 2;
    }
    if (kernel == 1) return hip_status(launch_gemv(q, s_x, packed, s_w, M, N, K, out, acc, s));
    if (kernel == 4) return hip_status(launch_skinny(q, s_x, packed, s_w, M, N, K, out, acc, s));
    if (forced_tile) return hip_status(launch_gemm_cfg(kernel - 16, q, s_x, packed, s_w, M, N, K, out, acc, s));
    return hip_status(launch_gemm(q, s_x, packed, s_w, M, N, K, out, acc, s));
}

BITNET_API int bitnet_linear(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                             int64_t M, int64_t N, int64_t K, float *y, int32_t *acc, void *stream) {
    return bitnet_linear_ex(q, s_x, packed, s_w, 0, M, N, K, nullptr, y, BITNET_F32, acc, 0, stream);
}

BITNET_API int bitnet_linear_select(const int8_t *q, const float *s_x, const uint8_t *packed,
                                    const float *s_w, int64_t M, int64_t N, int64_t K, float *y,
                                    int32_t *acc, int kernel, void *stream) {
    return bitnet_linear_ex(q, s_x, packed, s_w, 0, M, N, K, nullptr, y, BITNET_F32, acc, kernel, stream);
}

// ----------------------------------------------------------------- grouped plans

static size_t plan_layout(int count, size_t desc_size, uint64_t blocks, uint64_t *desc_off,
                          uint64_t *table_off) {
    *desc_off = sizeof(PlanHeader);
    *table_off = *desc_off + (uint64_t)count * desc_size;
    *table_off = (*table_off + 15) & ~(uint64_t)15;
    return (size_t)(*table_off + blocks * sizeof(BlockEntry));
}

// A plan whose problems all have M == 1 runs the GEMV (q staged in LDS); any M > 1
// makes it run the MFMA decode kernel, which reads each weight once for all M tokens.
// Problems with group-wise weight scales (w_group below K) make the whole plan run the
// kernels' group-wise paths: the GEMV's (one token per workgroup) when every M is 1,
// else the MFMA decode kernel's (BITNET_GROUPS_MFMA = 0: the GEMV's with kGemvGroupsMT
// tokens per workgroup, which reads the weights once per kGemvGroupsMT tokens).
#ifndef BITNET_GROUPS_MFMA
#define BITNET_GROUPS_MFMA 1
#endif
static bool desc_groups(const bitnet_linear_desc &d) { return d.w_group > 0 && d.w_group < d.K; }

static uint32_t linear_variant(const bitnet_linear_desc *d, int count) {
    for (int i = 0; i < count; ++i) {
        if (desc_groups(d[i])) {
            for (int j = 0; j < count; ++j)
                if (d[j].M > 1) return BITNET_GROUPS_MFMA ? kVariantMfmaGroups : kVariantGemvGroupsMT;
            return kVariantGemvGroups;
        }
    }
    for (int i = 0; i < count; ++i)
        if (d[i].M > 1) return kVariantMfma;
    return kVariantGemv;
}

static uint64_t linear_blocks(const bitnet_linear_desc &d, uint32_t variant) {
    if (variant == kVariantMfma || variant == kVariantMfmaGroups) {
        const uint64_t rows = skinny_grouped_rows_per_block();
        return ((uint64_t)d.N + rows - 1) / rows;
    }
    const uint64_t rows = gemv_grouped_rows_per_block();
    const uint64_t mt = variant == kVariantGemvGroupsMT ? kGemvGroupsMT : 1;
    return ((uint64_t)d.N + rows - 1) / rows * (((uint64_t)d.M + mt - 1) / mt);
}

// The output options of a descriptor: y's dtype and alignment, the bias.
static int check_desc_output(const void *y, int32_t y_dtype, const float *bias) {
    if (y_dtype != BITNET_F32 && y_dtype != BITNET_BF16) return fail(BITNET_ERR_ARG, "unknown output dtype");
    if (!aligned(y, y_dtype == BITNET_BF16 ? 2 : 4)) return fail(BITNET_ERR_ALIGN, "y must be aligned to its element size");
    if (bias && !aligned(bias, 4)) return fail(BITNET_ERR_ALIGN, "bias must be 4-byte aligned");
    return BITNET_OK;
}

static int check_linear_desc(const bitnet_linear_desc &d) {
    int st = check_dims(d.M, d.N, d.K);
    if (st) return st;
    if (!d.q || !d.s_x || !d.packed || !d.s_w || !d.y) return fail(BITNET_ERR_NULL, "null pointer");
    if (!aligned(d.s_x, 4) || !aligned(d.s_w, 4) || (d.acc && !aligned(d.acc, 4)))
        return fail(BITNET_ERR_ALIGN, "s_x, s_w and acc must be 4-byte aligned");
    st = check_desc_output(d.y, d.y_dtype, d.bias);
    if (st) return st;
    if (d.M < 1 || d.M > kGemvMaxM || d.N < 1) return fail(BITNET_ERR_SHAPE, "grouped linear needs 1 <= M <= 16, N >= 1");
    if (!linear_fast(d.q, d.packed, d.K)) return fail(BITNET_ERR_ALIGN, "grouped linear needs K % 64 == 0 and 16-byte aligned q/packed");
    if (d.w_group < 0 || (d.w_group > 0 && (d.K % d.w_group != 0 || (desc_groups(d) && d.w_group % 64 != 0))))
        return fail(BITNET_ERR_SHAPE, "w_group must be 0, K, or a multiple of 64 dividing K");
    return BITNET_OK;
}

static int check_fused_desc(const bitnet_fused_desc &d) {
    int st = check_dims(d.M, d.N, d.K);
    if (st) return st;
    if (d.M != 1 || d.N < 1) return fail(BITNET_ERR_SHAPE, "fused linear needs M == 1, N >= 1");
    if (d.weight_fmt != 0 && d.weight_fmt != BITNET_FMT_BITPLANES) return fail(BITNET_ERR_ARG, "unknown weight format");
    if (d.weight_fmt == BITNET_FMT_BITPLANES) {
        if (d.norm_gain || d.x_f32 || d.packed_up)
            return fail(BITNET_ERR_ARG, "bitplane weights take plain rows only (no norm_gain, x_f32 or packed_up)");
        if (d.K > bits_max_k(BITNET_FMT_BITPLANES)) return fail(BITNET_ERR_SHAPE, "bitplane rows need K <= 51584");
    }
    if (d.x_f32) {
        if (d.x || d.norm_gain) return fail(BITNET_ERR_ARG, "an fp32 row takes no x and no norm_gain");
        if (!aligned(d.x_f32, 16)) return fail(BITNET_ERR_ALIGN, "x_f32 must be 16-byte aligned");
    } else if (!d.x) {
        return fail(BITNET_ERR_NULL, "null pointer");
    }
    if (d.packed_up || d.s_w_up) {
        if (!d.packed_up || !d.s_w_up) return fail(BITNET_ERR_NULL, "packed_up and s_w_up go together");
        if (d.x_f32 || d.acc) return fail(BITNET_ERR_ARG, "a gate / up pair takes x (bf16) and no acc");
        if (!aligned(d.packed_up, 16) || !aligned(d.s_w_up, 4))
            return fail(BITNET_ERR_ALIGN, "packed_up must be 16-byte aligned, s_w_up 4-byte");
    }
    if (!d.packed || !d.s_w || !d.y) return fail(BITNET_ERR_NULL, "null pointer");
    if (d.K > gemv_fused_max_k()) return fail(BITNET_ERR_SHAPE, "fused linear needs K <= 52224");
    if (d.K % 64 != 0 || !aligned(d.x, 16) || !aligned(d.packed, 16) || (d.q && !aligned(d.q, 16)))
        return fail(BITNET_ERR_ALIGN, "fused linear needs K % 64 == 0 and 16-byte aligned x, packed and q");
    if (!aligned(d.s_w, 4) || (d.acc && !aligned(d.acc, 4)) || (d.s_x && !aligned(d.s_x, 4)))
        return fail(BITNET_ERR_ALIGN, "s_w, acc and s_x must be 4-byte aligned");
    st = check_desc_output(d.y, d.y_dtype, d.bias);
    if (st) return st;
    if (d.weight_fmt == BITNET_FMT_BITPLANES && (d.bias || d.y_dtype != BITNET_F32))
        return fail(BITNET_ERR_ARG, "bitplane weights take no bias and an fp32 y");
    if (d.packed_up && d.bias) return fail(BITNET_ERR_ARG, "a gate / up pair takes no bias");
    if (d.norm_gain) {
        if (!aligned(d.norm_gain, 16)) return fail(BITNET_ERR_ALIGN, "norm_gain must be 16-byte aligned");
        if (!(d.norm_eps >= 0.0f) || d.norm_eps > 3.4e38f) return fail(BITNET_ERR_ARG, "norm_eps must be finite and >= 0");
    }
    return BITNET_OK;
}

static int check_quant_desc(const bitnet_quant_desc &d) {
    int st = check_dims(d.M, 1, d.K);
    if (st) return st;
    if (d.M < 1) return fail(BITNET_ERR_SHAPE, "grouped quant needs M >= 1");
    if (!d.x || !d.q || !d.s_x) return fail(BITNET_ERR_NULL, "null pointer");
    if (d.K % 8 != 0 || !aligned(d.x, 16) || !aligned(d.q, 16) || !aligned(d.s_x, 4))
        return fail(BITNET_ERR_ALIGN, "grouped quant needs K % 8 == 0 and 16-byte aligned x/q");
    return BITNET_OK;
}

BITNET_API size_t bitnet_grouped_plan_bytes(int count, int is_linear, const void *descs) {
    if (count <= 0 || !descs) return 0;
    uint64_t blocks = 0, a, b;
    if (is_linear) {
        const bitnet_linear_desc *d = (const bitnet_linear_desc *)descs;
        const uint32_t variant = linear_variant(d, count);
        for (int i = 0; i < count; ++i) blocks += (d[i].M > 0 && d[i].N > 0) ? linear_blocks(d[i], variant) : 0;
        return plan_layout(count, sizeof(LinearDescDev), blocks, &a, &b);
    }
    const bitnet_quant_desc *d = (const bitnet_quant_desc *)descs;
    for (int i = 0; i < count; ++i) blocks += d[i].M > 0 ? (uint64_t)d[i].M : 0;
    return plan_layout(count, sizeof(QuantDescDev), blocks, &a, &b);
}

BITNET_API int bitnet_grouped_plan_linear(const bitnet_linear_desc *descs, int count, void *plan_host,
                                          size_t plan_bytes) {
    if (!descs || !plan_host) return fail(BITNET_ERR_NULL, "null pointer");
    if (count <= 0) return fail(BITNET_ERR_SHAPE, "count must be positive");
    uint64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        int st = check_linear_desc(descs[i]);
        if (st) return st;
    }
    const uint32_t variant = linear_variant(descs, count);
    for (int i = 0; i < count; ++i) blocks += linear_blocks(descs[i], variant);
    if (blocks >= ((uint64_t)1 << 31)) return fail(BITNET_ERR_SHAPE, "too many blocks");
    uint64_t doff, toff;
    const size_t need = plan_layout(count, sizeof(LinearDescDev), blocks, &doff, &toff);
    if (plan_bytes < need) return fail(BITNET_ERR_ARG, "plan buffer too small");
    uint8_t *p = (uint8_t *)plan_host;
    memset(p, 0, need);
    PlanHeader *h = (PlanHeader *)p;
    h->magic = kPlanMagic;
    h->kind = kPlanLinear;
    h->count = (uint32_t)count;
    h->total_blocks = (uint32_t)blocks;
    h->block_threads = gemv_grouped_threads();
    h->variant = variant;
    if (variant == kVariantMfma || variant == kVariantMfmaGroups) {
        h->rows_per_block = skinny_grouped_rows_per_block();
        for (int i = 0; i < count; ++i)
            h->lds_bytes = std::max(h->lds_bytes, skinny_grouped_lds_bytes(descs[i].M, descs[i].K, variant == kVariantMfmaGroups));
    } else {
        h->rows_per_block = gemv_grouped_rows_per_block();
        // each descriptor is staged by the path its own scales take (group-wise
        // descriptors keep one more dword per chunk, so they segment K sooner)
        const int mt = variant == kVariantGemvGroupsMT ? kGemvGroupsMT : 1;
        for (int i = 0; i < count; ++i)
            h->lds_bytes = std::max(h->lds_bytes, gemv_grouped_lds_bytes(descs[i].K, desc_groups(descs[i]), mt));
    }
    h->desc_offset = doff;
    h->table_offset = toff;
    h->total_bytes = need;
    for (int i = 0; i < count; ++i)
        if (desc_groups(descs[i]) && descs[i].acc) h->flags |= kPlanFlagGroupAcc;
    LinearDescDev *dd = (LinearDescDev *)(p + doff);
    BlockEntry *tb = (BlockEntry *)(p + toff);
    for (int i = 0; i < count; ++i) {
        const bitnet_linear_desc &d = descs[i];
        dd[i] = LinearDescDev{d.q, d.s_x, d.packed, d.s_w, d.y, d.acc, (int32_t)d.M, (int32_t)d.N, (int32_t)d.K,
                              (int32_t)d.w_group, d.bias, d.y_dtype == BITNET_BF16 ? 1 : 0, 0};
    }
    // Workgroups are dispatched roughly in table order: put the longest ones (largest
    // K, i.e. most bytes per row) first so that the short ones fill the tail.
    std::vector<int> order(count);
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return descs[a].K > descs[b].K; });
    uint64_t b = 0;
    for (int i : order) {
        const uint64_t nb = linear_blocks(descs[i], variant);
        for (uint64_t j = 0; j < nb; ++j) tb[b++] = BlockEntry{(uint32_t)i, (uint32_t)j};
    }
    return BITNET_OK;
}

BITNET_API int bitnet_grouped_plan_quant(const bitnet_quant_desc *descs, int count, void *plan_host,
                                         size_t plan_bytes) {
    if (!descs || !plan_host) return fail(BITNET_ERR_NULL, "null pointer");
    if (count <= 0) return fail(BITNET_ERR_SHAPE, "count must be positive");
    uint64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        int st = check_quant_desc(descs[i]);
        if (st) return st;
        blocks += (uint64_t)descs[i].M;
    }
    if (blocks >= ((uint64_t)1 << 31)) return fail(BITNET_ERR_SHAPE, "too many blocks");
    uint64_t doff, toff;
    const size_t need = plan_layout(count, sizeof(QuantDescDev), blocks, &doff, &toff);
    if (plan_bytes < need) return fail(BITNET_ERR_ARG, "plan buffer too small");
    uint8_t *p = (uint8_t *)plan_host;
    memset(p, 0, need);
    PlanHeader *h = (PlanHeader *)p;
    h->magic = kPlanMagic;
    h->kind = kPlanQuant;
    h->count = (uint32_t)count;
    h->total_blocks = (uint32_t)blocks;
    h->block_threads = 256;
    h->desc_offset = doff;
    h->table_offset = toff;
    h->total_bytes = need;
    QuantDescDev *dd = (QuantDescDev *)(p + doff);
    BlockEntry *tb = (BlockEntry *)(p + toff);
    uint64_t b = 0;
    for (int i = 0; i < count; ++i) {
        const bitnet_quant_desc &d = descs[i];
        dd[i] = QuantDescDev{d.x, d.q, d.s_x, (int32_t)d.M, (int32_t)d.K};
        for (int64_t j = 0; j < d.M; ++j) tb[b++] = BlockEntry{(uint32_t)i, (uint32_t)j};
    }
    return BITNET_OK;
}

static uint64_t fused_blocks(const bitnet_fused_desc &d) {
    // a gate / up pair takes both matrices' rows in each block: half the rows of each
    const uint64_t rows = (d.weight_fmt == BITNET_FMT_BITPLANES ? bits_fused_rows_per_block()
                                                                 : gemv_fused_rows_per_block()) /
                          (d.packed_up ? 2 : 1);
    return ((uint64_t)d.N + rows - 1) / rows;
}

BITNET_API size_t bitnet_grouped_plan_fused_bytes(int count, const bitnet_fused_desc *descs) {
    if (count <= 0 || !descs) return 0;
    uint64_t blocks = 0, a, b;
    for (int i = 0; i < count; ++i) blocks += descs[i].N > 0 ? fused_blocks(descs[i]) : 0;
    return plan_layout(count, sizeof(FusedDescDev), blocks, &a, &b);
}

BITNET_API int bitnet_grouped_plan_fused(const bitnet_fused_desc *descs, int count, void *plan_host,
                                         size_t plan_bytes) {
    if (!descs || !plan_host) return fail(BITNET_ERR_NULL, "null pointer");
    if (count <= 0) return fail(BITNET_ERR_SHAPE, "count must be positive");
    uint64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        int st = check_fused_desc(descs[i]);
        if (st) return st;
        if (descs[i].weight_fmt != descs[0].weight_fmt)
            return fail(BITNET_ERR_ARG, "every descriptor of a plan needs the same weight format");
        blocks += fused_blocks(descs[i]);
    }
    if (blocks >= ((uint64_t)1 << 31)) return fail(BITNET_ERR_SHAPE, "too many blocks");
    uint64_t doff, toff;
    const size_t need = plan_layout(count, sizeof(FusedDescDev), blocks, &doff, &toff);
    if (plan_bytes < need) return fail(BITNET_ERR_ARG, "plan buffer too small");
    uint8_t *p = (uint8_t *)plan_host;
    memset(p, 0, need);
    PlanHeader *h = (PlanHeader *)p;
    h->magic = kPlanMagic;
    h->kind = kPlanFused;
    h->count = (uint32_t)count;
    h->total_blocks = (uint32_t)blocks;
    h->block_threads = gemv_fused_threads();
    h->rows_per_block = gemv_fused_rows_per_block();
    const bool planes = descs[0].weight_fmt == BITNET_FMT_BITPLANES;
    h->variant = 0;   // mask of the prologues in use
    for (int i = 0; i < count; ++i) {
        if (descs[i].norm_gain) h->variant |= kFusedProNorm;
        if (descs[i].x_f32 || descs[i].packed_up) h->variant |= kFusedProSwiglu;
    }
    if (planes) {
        h->variant = kFusedBitplanes;
        h->rows_per_block = bits_fused_rows_per_block();
    }
    for (int i = 0; i < count; ++i)
        h->lds_bytes = std::max(h->lds_bytes, planes ? bits_fused_lds_bytes(descs[i].K) : gemv_grouped_lds_bytes(descs[i].K));
    h->desc_offset = doff;
    h->table_offset = toff;
    h->total_bytes = need;
    FusedDescDev *dd = (FusedDescDev *)(p + doff);
    BlockEntry *tb = (BlockEntry *)(p + toff);
    for (int i = 0; i < count; ++i) {
        const bitnet_fused_desc &d = descs[i];
        dd[i] = FusedDescDev{d.x, d.packed, d.s_w, d.y, d.acc, d.q, d.s_x, (int32_t)d.M, (int32_t)d.N, (int32_t)d.K, 0,
                             d.norm_gain, d.norm_gain ? d.norm_eps : 0.0f, 0, d.x_f32, d.packed_up, d.s_w_up,
                             d.bias, d.y_dtype == BITNET_BF16 ? 1 : 0, 0};
    }
    // longest rows first, as for linear plans
    std::vector<int> order(count);
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return descs[a].K > descs[b].K; });
    uint64_t b = 0;
    for (int i : order) {
        const uint64_t nb = fused_blocks(descs[i]);
        for (uint64_t j = 0; j < nb; ++j) tb[b++] = BlockEntry{(uint32_t)i, (uint32_t)j};
    }
    return BITNET_OK;
}

static int check_plan(const void *plan_host, const void *plan_dev, uint32_t kind) {
    if (!plan_host || !plan_dev) return fail(BITNET_ERR_NULL, "null plan");
    if (!aligned(plan_dev, 16)) return fail(BITNET_ERR_ALIGN, "device plan must be 16-byte aligned");
    const PlanHeader *h = (const PlanHeader *)plan_host;
    if (h->magic != kPlanMagic || h->kind != kind) return fail(BITNET_ERR_ARG, "not a plan of this kind");
    return BITNET_OK;
}

BITNET_API int bitnet_linear_grouped(const void *plan_host, const void *plan_dev, void *stream) {
    int st = check_plan(plan_host, plan_dev, kPlanLinear);
    if (st) return st;
    const PlanHeader *h = (const PlanHeader *)plan_host;
    if (h->total_blocks == 0) return BITNET_OK;
    if (h->variant == kVariantMfma || h->variant == kVariantMfmaGroups)
        return hip_status(launch_skinny_grouped(plan_dev, h->total_blocks, h->lds_bytes, h->variant == kVariantMfmaGroups,
                                                (h->flags & kPlanFlagGroupAcc) != 0, (hipStream_t)stream));
    if (h->variant != kVariantGemv && h->variant != kVariantGemvGroups && h->variant != kVariantGemvGroupsMT)
        return fail(BITNET_ERR_ARG, "not a plan of this kind");
    return hip_status(launch_gemv_grouped(plan_dev, h->total_blocks, h->lds_bytes, h->variant,
                                          (hipStream_t)stream));
}

BITNET_API int bitnet_linear_fused_grouped(const void *plan_host, const void *plan_dev, void *stream) {
    int st = check_plan(plan_host, plan_dev, kPlanFused);
    if (st) return st;
    const PlanHeader *h = (const PlanHeader *)plan_host;
    if (h->total_blocks == 0) return BITNET_OK;
    if (h->variant == kFusedBitplanes)
        return hip_status(launch_bits_fused_grouped(plan_dev, h->total_blocks, h->lds_bytes, (hipStream_t)stream));
    if (h->variant > kFusedProMask) return fail(BITNET_ERR_ARG, "not a plan of this kind");
    return hip_status(launch_gemv_fused_grouped(plan_dev, h->total_blocks, h->lds_bytes, h->variant,
                                                (hipStream_t)stream));
}

BITNET_API int bitnet_quant_act_grouped(const void *plan_host, const void *plan_dev, void *stream) {
    int st = check_plan(plan_host, plan_dev, kPlanQuant);
    if (st) return st;
    const PlanHeader *h = (const PlanHeader *)plan_host;
    if (h->total_blocks == 0) return BITNET_OK;
    return hip_status(launch_quant_act_grouped(plan_dev, h->total_blocks, (hipStream_t)stream));
}

}  // extern "C"
