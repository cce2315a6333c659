/*
 * bitnet.h -- C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear forward.
 *
 * The operation (pages: "BitNet 深度拆解……" on chenxutan.com, sec. 2.2
 * absmean / absmax quantization, sec. 2.3 rescale, sec. 3.1 BitLinear.forward,
 * sec. 3.3 INT2 packing; "1-bit推理框架bitnet.cpp实测……" on 0539edu.com,
 * sec. 2.1 RoundClip):
 *
 *   s_w      = mean |W|                                   (per tensor)
 *   t[n][k]  = clamp(round_half_even(W[n][k] / (s_w + eps)), -1, 1)
 *   s_x[m]   = max_k |x[m][k]|                             (per token)
 *   q[m][k]  = clamp(round_half_even(127 * x[m][k] / s_x[m]), -127, 127)
 *   acc[m][n]= sum_k q[m][k] * t[n][k]                     (exact int32)
 *   y[m][n]  = acc[m][n] * s_x[m] * s_w / 127               (fp32)
 *
 * Layouts (all row-major, K is the contiguous dimension):
 *   W       fp32  [N][K]     (nn.Linear weight: out_features x in_features)
 *   packed  uint8 [N][K/4]   byte (n, j) holds weights (n, 4j+i), i = 0..3, in
 *                            bits 2i..2i+1 as code t + 1 (0, 1, 2); a code of 3
 *                            is never written and is read as weight +2
 *   x       bf16  [M][K]     raw bit patterns (uint16)
 *   q       int8  [M][K],  s_x fp32 [M],  s_w fp32 [1]
 *   y       fp32  [M][N],  acc int32 [M][N]
 *
 * Memory and execution
 *   Every pointer argument marked (device) is device memory on the current HIP
 *   device; scales stay on the device, so consecutive calls need no host
 *   synchronisation.  The caller owns every buffer; the library allocates no
 *   memory and keeps no state between calls.  Work is enqueued asynchronously
 *   on `stream` (a hipStream_t, NULL = the default stream); buffers must stay
 *   valid until that work has completed.  Calls on different streams may run
 *   concurrently as long as their output buffers do not overlap.
 *
 * Errors
 *   Arguments are checked on the host before anything is enqueued; a failed
 *   check returns a status and enqueues nothing.  A launch failure reported by
 *   the runtime returns BITNET_ERR_HIP (the runtime's message is available
 *   from bitnet_last_error()).  Faults during execution surface at the
 *   caller's next synchronisation.  Inputs are assumed finite (non-finite
 *   inputs give unspecified values, never out-of-bounds accesses).
 *
 * Sizes: M, N, K are int64_t; K must be positive and a multiple of 4; M == 0 or
 * N == 0 is a successful no-op.  Fast kernels are used when K % 64 == 0 and the
 * q / packed / x base pointers are 16-byte aligned; other valid inputs take a
 * slower general kernel with identical results.
 */
#ifndef BITNET_H
#define BITNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(BITNET_BUILD)
#define BITNET_API __attribute__((visibility("default")))
#else
#define BITNET_API
#endif

typedef enum bitnet_status {
    BITNET_OK = 0,
    BITNET_ERR_NULL = 1,   /* a required pointer is NULL                      */
    BITNET_ERR_SHAPE = 2,  /* negative size, K <= 0, K % 4 != 0, bad count    */
    BITNET_ERR_ALIGN = 3,  /* a pointer the call requires aligned is not      */
    BITNET_ERR_HIP = 4,    /* the HIP runtime reported an error               */
    BITNET_ERR_ARG = 5     /* other invalid argument (workspace too small,
                              plan not made by bitnet_grouped_plan, ...)       */
} bitnet_status;

/* Human-readable name of a status code (static string, never NULL). */
BITNET_API const char *bitnet_status_str(int status);

/* Message of the last BITNET_ERR_HIP / BITNET_ERR_ARG on the calling thread
 * ("" if none). */
BITNET_API const char *bitnet_last_error(void);

/* ABI version (major * 100 + minor). */
BITNET_API int bitnet_version(void);

/* ---------------------------------------------------------------------------
 * Weight ternarization and packing (offline step).
 * Pages: chenxutan.com sec. 2.2 (absmean_quantize) and sec. 3.3 (pack_ternary);
 * 0539edu.com sec. 2.1 (scale = mean|w|, RoundClip to [-1, 1]).
 *
 *   w          (device) fp32 [N][K], 4-byte aligned
 *   eps        added to s_w before dividing (the configurations use 1e-5)
 *   packed     (device) uint8 [N][K/4], output
 *   s_w        (device) fp32 [1], output: mean |W| rounded once to fp32
 *   workspace  (device) at least bitnet_pack_workspace_bytes(N, K) bytes,
 *              8-byte aligned; holds per-row float64 sums during the call
 *
 * s_w is formed in float64: each row summed in increasing k, the row sums
 * added in increasing n, then one rounding to fp32; d = s_w + eps and w / d are
 * single binary32 operations (round to nearest even), so the result is
 * reproducible bit for bit.  N == 0 writes s_w = 0.
 * ------------------------------------------------------------------------- */
BITNET_API size_t bitnet_pack_workspace_bytes(int64_t N, int64_t K);
BITNET_API int bitnet_pack_weights(const float *w, int64_t N, int64_t K, float eps,
                                   uint8_t *packed, float *s_w,
                                   void *workspace, size_t workspace_bytes,
                                   void *stream);

/* ---------------------------------------------------------------------------
 * The same packing for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the
 * float64 row sums go to a scratch array the library holds, one copy per GPU,
 * allocated when the library is loaded and kept until the process ends; the
 * call itself allocates nothing.
 *
 *   w, eps, packed, s_w   as bitnet_pack_weights; results are bit-identical
 *   N                     at most BITNET_PACK_NOALLOC_MAX_ROWS (262144 rows,
 *                         2 MiB of scratch per GPU), else BITNET_ERR_SHAPE
 *                         before anything is enqueued
 *   stream                a stream of the current device (hipSetDevice)
 *
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap
 * in time on one GPU (different streams, or threads without ordering) race and
 * may give wrong s_w.  Calls ordered on one stream are safe.  The row sums are
 * fully written before they are read, so nothing needs clearing between calls.
 * ------------------------------------------------------------------------- */
#define BITNET_PACK_NOALLOC_MAX_ROWS 262144
BITNET_API int bitnet_pack_weights_noalloc(const float *w, int64_t N, int64_t K, float eps,
                                           uint8_t *packed, float *s_w, void *stream);

/* ---------------------------------------------------------------------------
 * Per-token absmax int8 activation quantization.
 * Page: chenxutan.com sec. 2.2 (absmax_quantize, 8 bits -> qmax 127).
 *
 *   x    (device) bf16 bit patterns [M][K]
 *   q    (device) int8 [M][K], output
 *   s_x  (device) fp32 [M], output: max_k |x[m][k]| (exact)
 *
 * q = round_half_even((127 * x) / s_x) with 127 * x exact and one correctly
 * rounded binary32 division, which equals the exact rounding of the real
 * quotient for every bf16 input; a row of zeros gives s_x = 0 and q = 0.
 * ------------------------------------------------------------------------- */
BITNET_API int bitnet_quant_act(const uint16_t *x, int64_t M, int64_t K,
                                int8_t *q, float *s_x, void *stream);

/* ---------------------------------------------------------------------------
 * RMSNorm of each token row followed by the same absmax int8 quantization of the
 * normalized row.  Page: chenxutan.com sec. 3.1 (the block normalizes the token
 * row with an RMSNorm kept in full precision before every projection; the linear
 * layer quantizes its input, sec. 2.2).
 *
 *   x     (device) bf16 bit patterns [M][K]
 *   gain  (device) fp32 [K], the norm's elementwise gain g
 *   eps   added to the mean square (finite, >= 0)
 *   q     (device) int8 [M][K], output;  s_x (device) fp32 [M], output
 *
 * The normalized value is the real number h = x g r, r = 1 / sqrt(mean_k x^2 +
 * eps).  Its codes are q = round_half_even(127 h / max|h|) = round_half_even(127
 * z / max|z|) with z = x g (r cancels), decided exactly (z and 127 z are exact in
 * float64 and the quotient is never rounded onto or across a half-integer); its
 * scale is s_x = max|h| = max|z| r, formed in float64 and rounded once to fp32
 * (the sum of squares in float64, in an order of the kernel's choosing).  A row
 * of zeros gives q = 0 and s_x = 0.  bitnet_linear then rescales with this s_x
 * as with any activation row.  Needs K % 8 == 0 and 16-byte aligned x, q and gain
 * (BITNET_ERR_SHAPE / BITNET_ERR_ALIGN).
 * ------------------------------------------------------------------------- */
BITNET_API int bitnet_rmsnorm_quant_act(const uint16_t *x, const float *gain, float eps,
                                        int64_t M, int64_t K, int8_t *q, float *s_x,
                                        void *stream);

/* ---------------------------------------------------------------------------
 * SwiGLU of the gate and up projections' outputs followed by the absmax int8
 * quantization of the result: the input row of the down projection.  Page:
 * chenxutan.com sec. 3.1 (the block's feed-forward part passes silu(gate(h)) *
 * up(h) to its down projection, silu(v) = v / (1 + e^-v); the down projection
 * quantizes its input on entry, sec. 2.2).
 *
 *   gate  (device) fp32 [M][K], the gate projection's output g
 *   up    (device) fp32 [M][K], the up projection's output u
 *   q     (device) int8 [M][K], output;  s_x (device) fp32 [M], output
 *
 * a = g u / (1 + e^-g) is evaluated in float64 and rounded once to fp32 (e^-g
 * with the device math library's float64 exp; a host float64 exp may differ in
 * its last bit, which moves a only where the float64 value lies within about
 * 2^-29 of an fp32 rounding boundary).  Then s_x = max|a| over the row and q =
 * round_half_even(127 a / s_x), decided exactly; a row of zeros gives q = 0 and
 * s_x = 0.  Inputs must give finite a.  Needs K % 8 == 0 and 16-byte aligned
 * gate, up and q (BITNET_ERR_SHAPE / BITNET_ERR_ALIGN).
 * ------------------------------------------------------------------------- */
BITNET_API int bitnet_swiglu_quant_act(const float *gate, const float *up, int64_t M, int64_t K,
                                       int8_t *q, float *s_x, void *stream);

/* ---------------------------------------------------------------------------
 * Ternary contraction with the fp32 rescale (BitLinear forward after the two
 * quantizations).  Pages: chenxutan.com sec. 2.3 (Y ~ (W_t . X_q) * act_scale *
 * beta) and sec. 3.1 (BitLinear.forward); the ternary product is a sign-select
 * add/subtract (chenxutan.com sec. 1).
 *
 *   q, s_x   (device) outputs of bitnet_quant_act
 *   packed   (device) uint8 [N][K/4], s_w (device) fp32 [1]: outputs of
 *            bitnet_pack_weights (any bytes are accepted; code 3 reads as +2)
 *   y        (device) fp32 [M][N], output
 *   acc      (device) int32 [M][N], output, or NULL to skip it
 *
 * acc is exact.  y is acc * s_x[m] * s_w / 127 evaluated as
 * fp32(acc * c_m) with c_m = (s_x[m] * s_w) / 127 in float64, i.e. within one
 * unit in the last place of the correctly rounded value.  M = 1 runs the
 * decode GEMV (4-bit dot products), 2 <= M <= 16 the MFMA decode kernel (int8
 * MFMA, all tokens in one pass over the weights), larger M the int8 MFMA GEMM.
 * ------------------------------------------------------------------------- */
BITNET_API int bitnet_linear(const int8_t *q, const float *s_x, const uint8_t *packed,
                             const float *s_w, int64_t M, int64_t N, int64_t K,
                             float *y, int32_t *acc, void *stream);

/* Same as bitnet_linear with the kernel chosen by the caller instead of by M
 * (for measuring the GEMV / GEMM crossover): kernel 0 = automatic, 1 = decode
 * GEMV (any M; M > 8 re-reads the weights once per 8 rows of q), 2 = MFMA GEMM,
 * 3 = general kernel, 4 = MFMA decode kernel (any M; the weights are read once
 * per 16 rows of q), 16 + i = MFMA GEMM with tile configuration i (0: 256 x 224,
 * 1: 256 x 80, 2: 256 x 128, 3: 128 x 128, 4: 64 x 128 rows x columns of y).
 * Kernels other than 0 and 3 need K % 64 == 0 and 16-byte aligned q / packed
 * (else BITNET_ERR_ALIGN); other values give BITNET_ERR_ARG. */
BITNET_API int bitnet_linear_select(const int8_t *q, const float *s_x, const uint8_t *packed,
                                    const float *s_w, int64_t M, int64_t N, int64_t K,
                                    float *y, int32_t *acc, int kernel, void *stream);

/* Output element types of bitnet_linear_ex. */
enum bitnet_dtype {
    BITNET_F32 = 0,   /* IEEE binary32                                     */
    BITNET_BF16 = 1   /* bfloat16 (upper half of binary32), uint16 storage */
};

/* ---------------------------------------------------------------------------
 * Weights with group-wise scales.  Pages: chenxutan.com sec. 3.1 (a weight_scale
 * per output channel), sec. 4.3 (group-wise quantization, groups of group_size
 * consecutive weights, commonly 128, each with its own scale); 0539edu.com sec.
 * 2.1 (scales per layer and per channel).
 *
 *   w       (device) fp32 [N][K]
 *   group   G: a multiple of 4 dividing K; G = K is one scale per output channel
 *   packed  (device) uint8 [N][K/4], output (the same 2-bit format)
 *   s_w     (device) fp32 [N][K/G], output
 *
 * Group g of row n (k = g G .. g G + G - 1) gets s_w[n][g] = fp32(mean |w|) (sum
 * in float64, k ascending) and codes clamp(rint(w / fl32(s_w[n][g] + eps)), -1, 1)
 * with binary32 operations, as bitnet_pack_weights does for the whole tensor.
 * ------------------------------------------------------------------------- */
BITNET_API int bitnet_pack_weights_grouped(const float *w, int64_t N, int64_t K, int64_t group,
                                           float eps, uint8_t *packed, float *s_w, void *stream);

/* bitnet_linear_select with the two epilogue options of the BitLinear forward
 * (chenxutan.com sec. 3.1 adds the layer's bias after the rescale; sec. 2.3 and
 * the bf16 activations of sec. 2.2 motivate a bf16 output for the next layer):
 *
 *   w_group  0: s_w is the tensor's one scale ([1]); else G with s_w [N][K/G]
 *            from bitnet_pack_weights_grouped (G = K: one scale per output channel)
 *   bias     (device) fp32 [N], added to every row of y, or NULL for none
 *   y        (device) [M][N] of y_dtype: BITNET_F32 or BITNET_BF16
 *   kernel   as for bitnet_linear_select (0 = automatic)
 *
 * With G = K: y[m][n] = fp32(acc * c_mn (+ bias[n])), c_mn = (s_x[m] s_w[n]) / 127
 * in float64, on every kernel.  With G < K: y[m][n] = fp32((sum_g acc_g s_w[n][g])
 * s_x[m] / 127 (+ bias[n])), acc_g the exact integer sum of group g and the sum over
 * groups in float64 (any order; the result is within 2^-23 |y| plus 2^-45 times
 * the sum of the terms' magnitudes of the ordered sum); acc is then sum_g acc_g.
 * Group-wise scales (G < K) run on the decode GEMV (kernel 1; needs G % 64 == 0
 * besides its usual conditions), the general kernel (3), or the pipelined GEMM
 * (kernel 2, or tiles 21 / 22) when acc is NULL, K % 128 == 0 and G is 64 or a
 * multiple of 128: there each group's exact integer sums are scaled into fp32
 * accumulators (y within 2^-23 |y| plus (K / G + 1) 2^-24 s_x / 127 times the sum
 * over groups of |acc_g s_w[n][g]|).  Kernel 0 picks the GEMM for M > 16 when it
 * can, else the GEMV (which re-reads the weights once per 8 rows of q); other
 * kernel ids, or the GEMM outside its conditions, give BITNET_ERR_ARG.  A w_group
 * that is not 0 or a multiple of 4 dividing K gives BITNET_ERR_SHAPE.
 *
 * y[m][n] = fp32(acc * c_m + bias[n]) with c_m = (s_x[m] * s_w) / 127, the
 * product and the sum taken in float64 and rounded once to fp32; a bf16 y is
 * that fp32 value rounded to nearest, ties to even (finite inputs only).  acc
 * is unchanged by the options.  bias must be 4-byte aligned, y aligned to its
 * element size (else BITNET_ERR_ALIGN); an unknown y_dtype or kernel gives
 * BITNET_ERR_ARG.  bitnet_linear and bitnet_linear_select are this call with
 * w_group = 0, bias = NULL and y_dtype = BITNET_F32. */
BITNET_API int bitnet_linear_ex(const int8_t *q, const float *s_x, const uint8_t *packed,
                                const float *s_w, int64_t w_group, int64_t M, int64_t N, int64_t K,
                                const float *bias, void *y, int y_dtype, int32_t *acc,
                                int kernel, void *stream);

/* ---------------------------------------------------------------------------
 * Grouped decode calls: many independent quant_act or linear problems in one
 * launch (a decode step has hundreds of small matrices; one launch each would
 * be dominated by dispatch gaps).  Same definitions and results as the single
 * calls, problem by problem.
 *
 * A plan is a byte image built on the host by bitnet_grouped_plan_*() from an
 * array of descriptors, copied by the caller to device memory once (e.g. with
 * hipMemcpy), and then launched any number of times.  The host image is needed
 * at launch for the grid size; the device copy is what the kernel reads.  The
 * pointers inside the descriptors are baked into the plan.
 *
 * Linear descriptors must have 1 <= M <= 16, K % 64 == 0 and 16-byte aligned
 * q / packed; quant descriptors K % 8 == 0 and 16-byte aligned x / q.  A linear
 * plan whose descriptors all have M = 1 runs the decode GEMV; if any has M > 1,
 * the whole plan runs the MFMA decode kernel (each weight read once for all M
 * tokens of its problem).
 * ------------------------------------------------------------------------- */
typedef struct bitnet_linear_desc {
    const int8_t *q;        /* (device) [M][K]   */
    const float *s_x;       /* (device) [M]      */
    const uint8_t *packed;  /* (device) [N][K/4] */
    const float *s_w;       /* (device) [1], or [N][K/w_group] */
    void *y;                /* (device) [M][N], fp32 or bf16 (y_dtype), 4- / 2-byte aligned */
    int32_t *acc;           /* (device) [M][N] or NULL */
    int64_t M, N, K;
    int64_t w_group;        /* weight-scale granularity as in bitnet_linear_ex: 0, K, or
                               a multiple of 64 dividing K (a plan holding any of the
                               latter runs the decode GEMV for all its problems) */
    const float *bias;      /* (device) [N] fp32, 4-byte aligned, or NULL: added after the
                               rescale, as in bitnet_linear_ex (page chenxutan.com sec. 3.1,
                               the bias of BitLinear) */
    int32_t y_dtype;        /* BITNET_F32 (0) or BITNET_BF16: y rounded once to fp32, then
                               to bf16 nearest-even, as in bitnet_linear_ex */
    int32_t reserved;       /* 0 */
} bitnet_linear_desc;

typedef struct bitnet_quant_desc {
    const uint16_t *x;      /* (device) [M][K] bf16 bits */
    int8_t *q;              /* (device) [M][K]  */
    float *s_x;             /* (device) [M]     */
    int64_t M, K;
} bitnet_quant_desc;

/* Size in bytes of the plan image for `count` descriptors. */
BITNET_API size_t bitnet_grouped_plan_bytes(int count, int is_linear, const void *descs);
/* Build a plan image into plan_host (plan_bytes >= bitnet_grouped_plan_bytes). */
BITNET_API int bitnet_grouped_plan_linear(const bitnet_linear_desc *descs, int count,
                                          void *plan_host, size_t plan_bytes);
BITNET_API int bitnet_grouped_plan_quant(const bitnet_quant_desc *descs, int count,
                                         void *plan_host, size_t plan_bytes);
/* Launch a plan: plan_host (host image) and plan_dev (device copy, 16-byte
 * aligned) must hold the same bytes. */
BITNET_API int bitnet_linear_grouped(const void *plan_host, const void *plan_dev, void *stream);
BITNET_API int bitnet_quant_act_grouped(const void *plan_host, const void *plan_dev, void *stream);

/* ---------------------------------------------------------------------------
 * Other weight encodings of the same product.
 *
 * BITNET_FMT_BINARY: b1.0 binary weights {-1, +1} (page chenxutan.com sec. 1 and
 * the b1.0 paragraph of sec. 2.1: the first BitNet's weights are binary, no zero).  bits (device) uint8 [N][K/8]:
 * weight k of row n is bit k % 8 of byte k / 8 (LSB first), set for +1.
 * BITNET_FMT_BITPLANES: the ternary weights as sign / mask bitplanes (the
 * untitled devpress.csdn.net summary on Microsoft's open BitNet framework, sec.
 * "三值量化：把乘法变成加减法": bitnet_linear over weight_sign and weight_mask).  planes (device) uint8 [N][K/32][8]: per 32
 * weights a little-endian mask word (bit i set: weight 32 c + i nonzero) then a
 * sign word (bit i set: -1; clear for zero weights).
 * ------------------------------------------------------------------------- */
#define BITNET_FMT_BINARY 1
#define BITNET_FMT_BITPLANES 2

/* Binary packing of w (device fp32 [N][K], 16-byte aligned, K % 32 == 0): t = +1
 * for w >= 0 (either zero), -1 below, and s_w = mean|w| over the tensor exactly as
 * bitnet_pack_weights forms it (float64 row sums in the workspace, same size rule).
 * NaN weights give -1.  bits (device) [N][K/8], 4-byte aligned. */
BITNET_API int bitnet_pack_weights_binary(const float *w, int64_t N, int64_t K, uint8_t *bits, float *s_w,
                                          void *workspace, size_t workspace_bytes, void *stream);

/* Sign / mask bitplanes of 2-bit packed weights (bitnet_pack_weights' layout),
 * K % 32 == 0, packed 8-byte aligned, planes (device) [N][K/32][8] 8-byte aligned.
 * Codes 0, 1, 2 become -1, 0, +1; a code 3 (never written by the packer) +1. */
BITNET_API int bitnet_pack_bitplanes(const uint8_t *packed, int64_t N, int64_t K, uint8_t *planes, void *stream);

/* acc[m][n] = sum_k q[m][k] t[n][k] (exact int32) and y = fp32(acc s_x[m] s_w / 127)
 * (formed as in bitnet_linear) for weights in format fmt.  K % 32 == 0.  kernel: 0
 * picks, 1 the general kernel (any M, any alignment), 2 the bit-serial GEMV (M == 1,
 * K % 128 == 0 for binary or K % 64 == 0 for bitplanes, K at most 57344 / 51584,
 * q and wbits 16-byte aligned; BITNET_ERR_ARG otherwise), 3 the bit-serial kernel for
 * several tokens (any M up to 65535: the weights are read once per 4 tokens for
 * binary, per 2 for bitplanes, fewer when one token's planes exceed 16 KiB; same K
 * divisibility and alignment, one token's planes within 64 KiB; BITNET_ERR_ARG
 * otherwise), 4 the matrix-core kernel (any M, the weights read once per 16 tokens:
 * bitplanes as their +1 and -1 planes, binary weights as their bits, each a set of
 * 0 / 1 bytes multiplied with q by int8 MFMAs; K % 64 == 0, q and wbits 16-byte
 * aligned; BITNET_ERR_ARG otherwise).  Kernel 0 takes 2 for one token and 4 for
 * more, else 3 when they apply.  acc may be NULL. */
BITNET_API int bitnet_linear_bits(const int8_t *q, const float *s_x, const uint8_t *wbits, int fmt,
                                  const float *s_w, int64_t M, int64_t N, int64_t K, float *y, int32_t *acc,
                                  int kernel, void *stream);

/* ---------------------------------------------------------------------------
 * Fused decode step: activation quantization and linear in one grouped launch
 * (pages: chenxutan.com sec. 2.2 absmax_quantize and sec. 3.1 BitLinear.forward,
 * whose forward quantizes the input on entry; sec. 5.3 item 4 on fusing the
 * steps around the product).  For every descriptor (one token, M = 1) the result
 * is bit-identical to bitnet_quant_act(x) followed by bitnet_linear(q, s_x, ...):
 * every workgroup of the problem quantizes the row itself while staging it, so no
 * q round trip through memory and no second launch are needed.  q and s_x are
 * optional outputs (written once, by one workgroup).
 *
 * Descriptors: M = 1, K % 64 == 0, K <= 52224 (the row's q fits one LDS
 * segment), x / packed / q 16-byte aligned.  Plans are built and launched like
 * the other grouped plans (host image + device copy).  A descriptor with
 * norm_gain set is bit-identical to bitnet_rmsnorm_quant_act(x, norm_gain,
 * norm_eps) followed by bitnet_linear instead (the RMSNorm before each projection
 * of chenxutan.com sec. 3.1, fused the same way; problems sharing a token row and
 * gain, such as q / k / v, each normalize it in their own workgroups).
 *
 * The two ends of the SwiGLU feed-forward part of chenxutan.com sec. 3.1
 * (down(silu(gate(h)) * up(h))):
 *  - a gate / up pair (packed_up and s_w_up set) computes both projections of the
 *    row in the same workgroups and writes y[n] = fp32(silu(y_gate[n]) y_up[n]),
 *    where y_gate / y_up are bitnet_linear's fp32 outputs of the two matrices (one
 *    rounding each) and the SwiGLU is evaluated in float64 and rounded once, as in
 *    bitnet_swiglu_quant_act; the pair takes x with or without norm_gain;
 *  - a descriptor with x_f32 quantizes that fp32 row like bitnet_quant_act does a
 *    bf16 row (s_x = max|x|, q = round_half_even(127 x / s_x) decided exactly), so
 *    bitnet_swiglu_quant_act(g, u) followed by bitnet_linear equals the pair's
 *    output fed through an x_f32 descriptor.
 * ------------------------------------------------------------------------- */
typedef struct bitnet_fused_desc {
    const uint16_t *x;      /* (device) [M][K] bf16 bits */
    const uint8_t *packed;  /* (device) [N][K/4] */
    const float *s_w;       /* (device) [1] */
    float *y;               /* (device) [M][N] */
    int32_t *acc;           /* (device) [M][N] or NULL */
    int8_t *q;              /* (device) [M][K] or NULL */
    float *s_x;             /* (device) [M] or NULL */
    int64_t M, N, K;
    const float *norm_gain; /* (device) [K] fp32, 16-byte aligned, or NULL: when set, the
                               row is RMSNorm-ed first (bitnet_rmsnorm_quant_act) */
    float norm_eps;         /* the norm's eps (finite, >= 0); ignored without norm_gain */
    const float *x_f32;     /* (device) [M][K] fp32, 16-byte aligned, or NULL: the input row
                               in fp32 instead of x (x and norm_gain NULL), such as the
                               SwiGLU output feeding a down projection */
    const uint8_t *packed_up; /* (device) [N][K/4], 16-byte aligned, or NULL: with s_w_up,
                               the problem is the gate (packed, s_w) / up (packed_up,
                               s_w_up) pair of a SwiGLU feed-forward part; acc must be NULL */
    const float *s_w_up;    /* (device) [1] */
    int32_t weight_fmt;     /* 0: packed holds 2-bit codes; BITNET_FMT_BITPLANES: packed holds
                               the sign / mask bitplanes [N][K/32][8] of the same weights (plain
                               rows only: no norm_gain, x_f32 or packed_up; K <= 51584).  Every
                               descriptor of a plan has the same format. */
    int32_t y_dtype;        /* BITNET_F32 (0) or BITNET_BF16 for y (2-byte aligned for bf16):
                               rounded once to fp32, then to bf16 nearest-even; 2-bit codes only */
    const float *bias;      /* (device) [N] fp32, 4-byte aligned, or NULL: added after the
                               rescale (page chenxutan.com sec. 3.1, the bias of BitLinear);
                               2-bit codes only, and not on a gate / up pair */
} bitnet_fused_desc;

BITNET_API size_t bitnet_grouped_plan_fused_bytes(int count, const bitnet_fused_desc *descs);
BITNET_API int bitnet_grouped_plan_fused(const bitnet_fused_desc *descs, int count,
                                         void *plan_host, size_t plan_bytes);
BITNET_API int bitnet_linear_fused_grouped(const void *plan_host, const void *plan_dev, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_H */
