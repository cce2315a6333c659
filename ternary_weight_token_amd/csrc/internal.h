// Host-side declarations shared by the launchers and the C ABI (not exported).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitnet {

// Output of the rescale epilogue (pages: chenxutan.com sec. 2.3 rescale, sec. 3.1
// forward with its optional bias): y = acc * c_m (+ bias[n]), c_m = (s_x * s_w) / 127,
// formed in float64 and rounded once to fp32; a bf16 output is that fp32 value
// rounded to nearest even.  w_group: granularity of the weight scales s_w (sec. 3.1
// weight_scale per output channel, sec. 4.3 groups): 0 = one scale for the tensor,
// K = one per output channel (s_w[n]), G = one per G consecutive weights of a row
// (s_w[n][k / G]).
struct OutSpec {
    void *y;             // fp32 or bf16, [M][N]
    const float *bias;   // [N] or nullptr
    int bf16;
    int w_group;
};

// The same output advanced by `elems` elements (a later row block of y).
__host__ __device__ inline OutSpec out_offset(const OutSpec &o, size_t elems) {
    return OutSpec{static_cast<char *>(o.y) + elems * (o.bf16 ? 2 : 4), o.bias, o.bf16, o.w_group};
}

// Plan image for grouped launches.
constexpr uint32_t kPlanMagic = 0xB17E7A01u;
constexpr uint32_t kPlanLinear = 1, kPlanQuant = 2, kPlanFused = 3;

// Linear plan variants: one block per (row block, token) running the GEMV, or one
// block per row block running the MFMA decode kernel for all tokens at once.
constexpr uint32_t kVariantGemv = 0, kVariantMfma = 1;
// ... and the GEMV with the group-wise-scale path, for plans with such weights: one
// token per workgroup, or (any M > 1 among them) up to kGemvGroupsMT tokens per
// workgroup, so that the weights are read once per kGemvGroupsMT tokens.
constexpr uint32_t kVariantGemvGroups = 2, kVariantGemvGroupsMT = 3;
constexpr int kGemvGroupsMT = 4;
// ... and the MFMA decode kernel with its group-wise path, for plans with such weights
// and any M > 1 (every problem once over its weights, all tokens at once; the plan's
// other problems take that path too, with one group of all of K).
constexpr uint32_t kVariantMfmaGroups = 4;
// Fused plan variants: a mask of what its problems use beyond the plain path (an
// RMSNorm; fp32 input rows or gate / up pairs, the two ends of SwiGLU); each mask
// has its own kernel, so a plan without them takes the kernel without that code.
constexpr uint32_t kFusedProNorm = 1, kFusedProSwiglu = 2, kFusedProMask = 3;
// a fused plan over bitplane weights (plain rows only) has this variant instead
constexpr uint32_t kFusedBitplanes = 4;

struct PlanHeader {            // 64 bytes
    uint32_t magic, kind, count, total_blocks;
    uint32_t block_threads, rows_per_block, lds_bytes, variant;
    uint64_t desc_offset, table_offset, total_bytes, flags;   // flags: kPlanFlag*
};
// a linear plan with group-wise scales where some such descriptor asks for int32 acc
constexpr uint64_t kPlanFlagGroupAcc = 1;

struct LinearDescDev {         // 80 bytes, device layout
    const int8_t *q; const float *s_x; const uint8_t *packed; const float *s_w;
    void *y; int32_t *acc;
    int32_t M, N, K, w_group;  // w_group as OutSpec::w_group
    const float *bias;         // [N] or null
    int32_t bf16, pad;         // y as bf16 when set
    __host__ __device__ OutSpec out() const { return OutSpec{y, bias, bf16, w_group}; }
};

struct QuantDescDev {          // 32 bytes
    const uint16_t *x; int8_t *q; float *s_x;
    int32_t M, K;
};

struct FusedDescDev {          // 128 bytes: (RMSNorm +) quantization + linear of one token row
    const uint16_t *x; const uint8_t *packed; const float *s_w;
    void *y; int32_t *acc; int8_t *q; float *s_x;
    int32_t M, N, K, pad;
    const float *gain; float eps; int32_t pad2;
    const float *xf;           // fp32 input row instead of x, or null
    const uint8_t *packed2;    // up projection of a gate / up pair (SwiGLU epilogue), or null
    const float *s_w2;
    const float *bias;         // [N] or null (not on pairs)
    int32_t bf16, pad3;        // y as bf16 when set
};

struct BlockEntry { uint32_t desc, local; };

// launchers (return hipError_t of the launch)
hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s_x,
                            hipStream_t st);
hipError_t launch_quant_act_grouped(const void *plan_dev, uint32_t blocks, hipStream_t st);
hipError_t launch_swiglu_quant(const float *g, const float *u, int64_t M, int64_t K, int8_t *q, float *s_x,
                               hipStream_t st);
hipError_t launch_rmsnorm_quant(const uint16_t *x, const float *g, float eps, int64_t M, int64_t K, int8_t *q,
                                float *s_x, hipStream_t st);
// s_w = mean |w| of the whole tensor (the row sums in rowsum, float64)
hipError_t launch_weight_scale(const float *w, int64_t N, int64_t K, float *s_w, double *rowsum, hipStream_t st);
// other weight encodings (bits.hip): b1.0 binary bits, sign / mask bitplanes
hipError_t launch_pack_binary(const float *w, int64_t N, int64_t K, uint8_t *bits, hipStream_t st);
hipError_t launch_pack_bitplanes(const uint8_t *packed, int64_t N, int64_t K, uint8_t *planes, hipStream_t st);
int64_t bits_max_k(int fmt);
uint32_t bits_fused_rows_per_block();
uint32_t bits_fused_lds_bytes(int64_t K);
hipError_t launch_bits_fused_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, hipStream_t st);
bool bits_fast_ok(int fmt, int64_t M, int64_t K, const void *q, const void *wbits);
bool bits_mt_ok(int fmt, int64_t K, const void *q, const void *wbits);   // several tokens per pass
bool bits_mfma_ok(int fmt, int64_t M, int64_t K, const void *q, const void *wbits);   // bitplanes on MFMA
hipError_t launch_linear_bits(const int8_t *q, const float *s_x, const uint8_t *wbits, int fmt, const float *s_w,
                              int64_t M, int64_t N, int64_t K, float *y, int32_t *acc, int kernel, hipStream_t st);
hipError_t launch_pack(const float *w, int64_t N, int64_t K, float eps, uint8_t *packed,
                       float *s_w, double *rowsum, hipStream_t st);
// Library-held row-sum scratch of the pack step (one copy per GPU, rows up to
// kPackScratchRows): its device address on the current device.
constexpr int64_t kPackScratchRows = (int64_t)1 << 18;
constexpr int kMaxScratchDevices = 64;
hipError_t pack_scratch(double **out);
hipError_t launch_pack_grouped(const float *w, int64_t N, int64_t K, int64_t G, float eps, uint8_t *packed,
                               float *s_w, hipStream_t st);
hipError_t launch_gemv(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                       int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st);
hipError_t launch_gemv_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, uint32_t variant,
                               hipStream_t st);
uint32_t gemv_grouped_lds_bytes(int64_t K, bool grp = false, int mt = 1);
hipError_t launch_gemv_fused_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, uint32_t pro,
                                     hipStream_t st);
int64_t gemv_fused_max_k();
uint32_t gemv_grouped_rows_per_block();
uint32_t gemv_fused_rows_per_block();
uint32_t gemv_fused_threads();
uint32_t gemv_grouped_threads();
double skinny_estimate_us(int64_t M, int64_t N, int64_t K);
double gemm_estimate_us(int64_t M, int64_t N, int64_t K);
hipError_t launch_skinny(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                         int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st);
hipError_t launch_skinny_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, bool grp, bool grp_acc,
                                 hipStream_t st);
uint32_t skinny_grouped_rows_per_block();
uint32_t skinny_grouped_lds_bytes(int64_t M, int64_t K, bool grp = false);
hipError_t launch_gemm(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                       int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st);
hipError_t launch_gemm_cfg(int cfg, const int8_t *q, const float *s_x, const uint8_t *packed,
                           const float *s_w, int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc,
                           hipStream_t st);
int gemm_config_count();
// pipelined persistent GEMM (gemm_pipe.hip); tn_force 0 = by its cost model, else 5 or 7
bool gemm_pipe_ok(int64_t M, int64_t N, int64_t K);
// group-wise scales (w_group < K) on the pipelined kernel: G = 64 or a multiple of 128
bool gemm_pipe_groups_ok(int64_t M, int64_t N, int64_t K, int64_t w_group);
int64_t gemm_pipe_rounds(int64_t M, int64_t N);   // tiles per busiest workgroup on 256 CUs
double gemm_pipe_estimate_us(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_pipe(int tn_force, const int8_t *q, const float *s_x, const uint8_t *packed,
                            const float *s_w, int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc,
                            hipStream_t st);
// measurement probes (probe.hip)
hipError_t launch_probe_stream_read(const void *buf, int64_t bytes, int64_t blocks, uint32_t key, uint32_t *sink,
                                    hipStream_t st);
hipError_t launch_probe_mfma_i8(int64_t blocks, int64_t iters, uint32_t key, uint32_t *sink, hipStream_t st);
double probe_mfma_i8_ops(int64_t blocks, int64_t iters);
hipError_t launch_linear_generic(const int8_t *q, const float *s_x, const uint8_t *packed,
                                 const float *s_w, int64_t M, int64_t N, int64_t K, const OutSpec &y,
                                 int32_t *acc, hipStream_t st);

}  // namespace bitnet
