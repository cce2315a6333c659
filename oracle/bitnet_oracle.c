/*
 * CPU oracle for the BitNet b1.58 BitLinear forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it is used by the tests, by the smoke check and by the
 * bench's CPU-baseline leg, and by nothing else.  It shares no code, header,
 * table or constant with the GPU library.
 *
 * It is written to be read against the pages, not to be fast: every function
 * is the plain definition, step by step, with no blocking, fusion or
 * reordering beyond what the definition states.  The only concession to speed
 * is an OpenMP "parallel for" over independent output rows, which changes no
 * arithmetic.
 *
 * Sources (page titles as printed on the pages):
 *  [P1] "BitNet 深度拆解：当大模型被压到 1.58 bit……" (chenxutan.com),
 *       sec. 2.2 (absmean / absmax quantization), sec. 2.3 (rescale with the
 *       two scale factors), sec. 3.1 (BitLinear.forward), sec. 3.3 (INT2
 *       packing, 4 weights per byte, code = w + 1, LSB first).
 *  [P3] untitled summary of Microsoft's open BitNet framework (devpress.csdn.net),
 *       sec. "三值量化：把乘法变成加减法" (bitnet_linear over weight_sign and
 *       weight_mask: the sign / mask bitplanes).
 *  [P5] "1-bit推理框架bitnet.cpp实测……" (0539edu.com), sec. 2.1
 *       (RoundClip(w / scale, -1, 1), scale = mean|w|).
 *
 * Readings where the pages are ambiguous (each is argued in the design notes):
 *  - weight scale s_w = mean|W| over the whole tensor ([P5] 2.1); the mean is
 *    formed in float64, row sums first (each row summed k = 0..K-1 in order),
 *    then the row sums added n = 0..N-1 in order, then one rounding to fp32;
 *  - ternary code: t = clamp(rint(w / (s_w + eps)), -1, 1) with s_w + eps and
 *    the quotient each one IEEE binary32 operation (the pages' tensors are
 *    fp32); rint is round-half-to-even, the rounding of torch.round in [P1];
 *  - activation code: q = clamp(RNE(127 * x / max|x_row|), -127, 127) where the
 *    quotient is the exact real number (computed in float64, which is exact
 *    for bf16 inputs, see the tests); an all-zero row gives q = 0, s_x = 0;
 *  - output y = acc * c with one rescale factor per token row and weight scale,
 *    c = (s_x * s_w) / 127 formed in float64 ([P1] 2.3 applies the two scale
 *    factors to the integer product; the /127 undoes the *127 of the activation
 *    code), then acc * c in float64 and one rounding to fp32;
 *  - a 2-bit field holding 3 (never written by the packer) decodes to +2;
 *  - the optional bias ([P1] 3.1 adds it after the rescale) joins the float64
 *    value before its one rounding to fp32; a bf16 output is that fp32 value
 *    rounded again, to nearest bf16, ties to even;
 *  - RMSNorm before quantization, group-wise weight scales and SwiGLU before the
 *    down projection: see the comments of their functions below.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* --- threads ------------------------------------------------------------ */

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* --- weights: absmean scale ([P1] 2.2 absmean_quantize, [P5] 2.1) -------- */

/* rowsum[n] = sum_k |W[n][k]| in float64, k ascending; returns s_w = fp32 of
 * (sum_n rowsum[n]) / (N*K), n ascending. */
float oracle_weight_scale(const float *w, int64_t N, int64_t K, double *rowsum) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double r = 0.0;
        for (int64_t k = 0; k < K; ++k) r += fabs((double)w[n * K + k]);
        rowsum[n] = r;
    }
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) total += rowsum[n];
    if (N * K == 0) return 0.0f;
    return (float)(total / (double)(N * K));
}

/* --- weights: ternary code and 2-bit packing ([P1] 3.3 pack_ternary) ---- */

/* t = clamp(rint(w / d), -1, 1) with d = fl32(s_w + eps). */
static int ternary_of(float w, float d) {
    float v = w / d;                 /* one binary32 division */
    float r = rintf(v);              /* half to even */
    if (r > 1.0f) r = 1.0f;
    if (r < -1.0f) r = -1.0f;
    return (int)r;
}

/* packed[n][j] holds weights (n, 4j .. 4j+3); weight 4j+i sits in bits
 * 2i..2i+1 as code t + 1.  K must be a multiple of 4 (no padding). */
void oracle_pack(const float *w, int64_t N, int64_t K, float eps,
                 float s_w, uint8_t *packed) {
    float d = s_w + eps;             /* one binary32 addition */
    int64_t KB = K / 4;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < KB; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                int t = ternary_of(w[n * K + 4 * j + i], d);
                unsigned code = (unsigned)(t + 1);
                byte |= code << (2 * i);
            }
            packed[n * KB + j] = (uint8_t)byte;
        }
    }
}

/* Group-wise scales ([P1] 3.1: a weight_scale per output channel; [P1] 4.3:
 * groups of group_size consecutive weights, each with its own scale; [P5] 2.1:
 * scales per channel): row n is cut into K / G groups of G consecutive k; group g
 * gets s = fp32(mean |w| over the group) (float64 sum, k ascending) and its codes
 * t = clamp(rint(w / fl32(s + eps)), -1, 1) as in oracle_pack.  G = K is one scale
 * per output channel.  s_w: [N][K / G]. */
void oracle_pack_grouped(const float *w, int64_t N, int64_t K, int64_t G, float eps,
                         float *s_w, uint8_t *packed) {
    const int64_t ng = K / G, KB = K / 4;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < ng; ++g) {
            double sum = 0.0;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) sum += fabs((double)w[n * K + k]);
            s_w[n * ng + g] = (float)(sum / (double)G);
        }
        for (int64_t j = 0; j < KB; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                const int64_t k = 4 * j + i;
                const float d = s_w[n * ng + k / G] + eps;
                const int t = ternary_of(w[n * K + k], d);
                byte |= (unsigned)(t + 1) << (2 * i);
            }
            packed[n * KB + j] = (uint8_t)byte;
        }
    }
}

/* Decode one weight from the packed layout (code - 1; code 3 -> +2). */
static int weight_at(const uint8_t *packed, int64_t KB, int64_t n, int64_t k) {
    unsigned byte = packed[n * KB + k / 4];
    unsigned code = (byte >> (2 * (k % 4))) & 3u;
    return (int)code - 1;
}

void oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *t) {
    int64_t KB = K / 4;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            t[n * K + k] = (int8_t)weight_at(packed, KB, n, k);
}

/* --- activations: absmax int8 ([P1] 2.2 absmax_quantize) ---------------- */

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void oracle_quant_act(const uint16_t *x, int64_t M, int64_t K,
                      int8_t *q, float *s_x) {
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = x + m * K;
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(bf16_to_float(row[k]));
            if (a > s) s = a;
        }
        s_x[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            if (s == 0.0f) { q[m * K + k] = 0; continue; }
            double v = (127.0 * (double)bf16_to_float(row[k])) / (double)s;
            double r = rint(v);      /* half to even */
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            q[m * K + k] = (int8_t)r;
        }
    }
}

/* The same absmax quantization ([P1] 2.2) of fp32 rows (the SwiGLU output that
 * feeds a down projection is fp32): s = max|x| (exact), q = RNE(127 x / s) with the
 * real quotient.  127 x is exact in float64 and the correctly rounded float64
 * quotient cannot create or cross a half-integer (see oracle_swiglu_quant), so the
 * codes are the exact rounding.  x: fp32 [M][K]. */
void oracle_quant_act_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *s_x) {
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k)
            if (fabsf(row[k]) > s) s = fabsf(row[k]);
        s_x[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            if (s == 0.0f) { q[m * K + k] = 0; continue; }
            double r = rint((127.0 * (double)row[k]) / (double)s);
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            q[m * K + k] = (int8_t)r;
        }
    }
}

/* --- RMSNorm before the activation quantization ([P1] 3.1) -------------- */

/* The block of [P1] 3.1 feeds its projections from an RMSNorm of the token row;
 * [P1] keeps the norm in full precision and quantizes its output inside the
 * linear layer (absmax, [P1] 2.2).  Here the norm's value is the real number
 *     h_k = x_k g_k r,   r = 1 / sqrt(mean_k(x_k^2) + eps),
 * and it is quantized like any activation row:
 *     s = max_k |h_k| = r max_k |x_k g_k|,   q_k = RNE(127 h_k / s).
 * r cancels in q_k = RNE(127 z_k / max|z|) with z_k = x_k g_k, which float64
 * holds exactly (8 + 24 significant bits); 127 z_k too, and the one rounding of
 * the quotient cannot create or cross a half-integer (127 z / max|z| is a ratio
 * of integers below 2^40 times powers of two, so it is either a tie exactly or
 * at least 2^-41 relatively away from one).  The scale s_x = fp32(max|z| r) is
 * formed in float64 with the sum of squares taken k = 0 .. K-1 in order.  An
 * all-zero row (max|z| = 0) gives q = 0 and s_x = 0.
 *   x: bf16 bits [M][K]; g: fp32 [K]; outputs q int8 [M][K], s_x fp32 [M]. */
void oracle_rmsnorm_quant(const uint16_t *x, const float *g, float eps, int64_t M, int64_t K,
                          int8_t *q, float *s_x) {
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = x + m * K;
        double mz = 0.0, ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double xv = (double)bf16_to_float(row[k]);
            const double z = xv * (double)g[k];
            if (fabs(z) > mz) mz = fabs(z);
            ss += xv * xv;
        }
        if (mz == 0.0) {
            s_x[m] = 0.0f;
            for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
            continue;
        }
        const double r = 1.0 / sqrt(ss / (double)K + (double)eps);
        s_x[m] = (float)(mz * r);
        for (int64_t k = 0; k < K; ++k) {
            const double z = (double)bf16_to_float(row[k]) * (double)g[k];
            double v = rint((127.0 * z) / mz);
            if (v > 127.0) v = 127.0;
            if (v < -127.0) v = -127.0;
            q[m * K + k] = (int8_t)v;
        }
    }
}

/* --- SwiGLU before the down projection's quantization ([P1] 3.1) -------- */

/* [P1] 3.1's block feeds its down projection with silu(gate(h)) * up(h): the
 * activation row of down is a_k = silu(g_k) u_k, g and u the fp32 outputs of the
 * gate and up projections, silu(v) = v / (1 + exp(-v)).  Here a_k is that real
 * value rounded once to fp32 (evaluated in float64 with the C library's exp), and
 * the row is quantized like any activation row: s = max_k |a_k| (exact), q_k =
 * RNE(127 a_k / s).  127 a_k is exact in float64 and the correctly rounded quotient
 * cannot create or cross a half-integer (the ratio of two fp32 values times 127
 * is either exactly one or at least 2^-32 relatively away), so the codes are the
 * exact rounding.  A row of zeros gives q = 0 and s_x = 0.
 *   g, u: fp32 [M][K]; outputs a fp32 [M][K] (or NULL), q int8 [M][K], s_x [M]. */
static float silu_mul(float g, float u) {
    const double gd = (double)g;
    return (float)((gd / (1.0 + exp(-gd))) * (double)u);
}

void oracle_swiglu_quant(const float *g, const float *u, int64_t M, int64_t K, float *a, int8_t *q,
                         float *s_x) {
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = silu_mul(g[m * K + k], u[m * K + k]);
            if (a) a[m * K + k] = v;
            if (fabsf(v) > s) s = fabsf(v);
        }
        s_x[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            if (s == 0.0f) { q[m * K + k] = 0; continue; }
            const double v = (double)silu_mul(g[m * K + k], u[m * K + k]);
            double r = rint((127.0 * v) / (double)s);
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            q[m * K + k] = (int8_t)r;
        }
    }
}

/* --- contraction and rescale ([P1] 2.3, 3.1 BitLinear.forward) ---------- */

/* acc[m][n] = sum_k q[m][k] * t[n][k]  (exact integer sum)
 * c_m       = (s_x[m] * s_w) / 127                       in float64 (s_x s_w is exact),
 * y[m][n]   = fp32( acc * c_m + bias[n] )                  in float64;
 * the bias is the layer's own bias, added after the rescale ([P1] 3.1, where
 * BitLinear.forward adds self.bias to the dequantized product).
 * acc and bias may be NULL (no bias: the sum has no second term). */
static double row_factor(float s_x, float s_w) {
    return ((double)s_x * (double)s_w) / 127.0;
}

void oracle_linear_bias(const int8_t *q, const float *s_x, const uint8_t *packed,
                        float s_w, const float *bias, int64_t M, int64_t N, int64_t K,
                        int32_t *acc, float *y) {
    int64_t KB = K / 4;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t a = 0;
            for (int64_t k = 0; k < K; ++k)
                a += (int64_t)q[m * K + k] * (int64_t)weight_at(packed, KB, n, k);
            if (acc) acc[m * N + n] = (int32_t)a;
            double v = (double)a * row_factor(s_x[m], s_w);
            if (bias) v = v + (double)bias[n];
            y[m * N + n] = (float)v;
        }
    }
}

/* Group-wise scales: acc_g[m][n] = sum over group g of q t (exact integer), and
 * y[m][n] = fp32( (sum_g acc_g s_w[n][g]) * s_x[m] / 127 (+ bias[n]) ), the sum
 * over g ascending, all in float64; acc[m][n] = sum_g acc_g (the whole-row
 * integer sum, for inspection).  acc and bias may be NULL.  A single group per
 * row (G = K: one scale per output channel) is the per-tensor rescale with the
 * row's own scale: y = fp32(acc * c + bias), c = (s_x[m] * s_w[n]) / 127. */
void oracle_linear_grouped(const int8_t *q, const float *s_x, const uint8_t *packed,
                           const float *s_w, int64_t G, const float *bias, int64_t M, int64_t N,
                           int64_t K, int32_t *acc, float *y) {
    const int64_t KB = K / 4, ng = K / G;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t total = 0;
            double v = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                int64_t a = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k)
                    a += (int64_t)q[m * K + k] * (int64_t)weight_at(packed, KB, n, k);
                total += a;
                v += (double)a * (double)s_w[n * ng + g];
            }
            if (acc) acc[m * N + n] = (int32_t)total;
            if (ng == 1) {
                v = (double)total * row_factor(s_x[m], s_w[n]);
            } else {
                v = v * (double)s_x[m];
                v = v / 127.0;
            }
            if (bias) v = v + (double)bias[n];
            y[m * N + n] = (float)v;
        }
    }
}

void oracle_linear(const int8_t *q, const float *s_x, const uint8_t *packed,
                   float s_w, int64_t M, int64_t N, int64_t K,
                   int32_t *acc, float *y) {
    oracle_linear_bias(q, s_x, packed, s_w, NULL, M, N, K, acc, y);
}

/* --- other weight encodings: b1.0 binary weights, sign / mask bitplanes --- */

/* Binary weights ([P1] 1 and the b1.0 paragraph of 2.1: the first BitNet's weights are
 * {-1, +1}, no zero).  The pages give no binarization rule; here t = +1 for
 * w >= 0 (either zero) and -1 for w < 0, with the same absmean scale s_w as the
 * ternary weights (oracle_weight_scale; mean |w| is also the scale that best fits
 * sign(W) in the least-squares sense).  Layout: row n holds K / 8 bytes, weight k
 * in byte k / 8, bit k % 8 (LSB first), set for +1.  K % 8 == 0. */
void oracle_pack_binary(const float *w, int64_t N, int64_t K, uint8_t *bits) {
    const int64_t KB = K / 8;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < KB; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 8; ++i)
                if (w[n * K + 8 * j + i] >= 0.0f) byte |= 1u << i;
            bits[n * KB + j] = (uint8_t)byte;
        }
    }
}

static int binary_at(const uint8_t *bits, int64_t K, int64_t n, int64_t k) {
    return ((bits[n * (K / 8) + k / 8] >> (k % 8)) & 1u) ? 1 : -1;
}

/* acc = sum_k q t (exact), y = fp32(acc c_m), c_m = (s_x s_w) / 127, as oracle_linear. */
void oracle_linear_binary(const int8_t *q, const float *s_x, const uint8_t *bits, float s_w, int64_t M,
                          int64_t N, int64_t K, int32_t *acc, float *y) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t a = 0;
            for (int64_t k = 0; k < K; ++k) a += (int64_t)q[m * K + k] * binary_at(bits, K, n, k);
            if (acc) acc[m * N + n] = (int32_t)a;
            y[m * N + n] = (float)((double)a * row_factor(s_x[m], s_w));
        }
    }
}

/* Sign / mask bitplanes ([P3], bitnet_linear with weight_sign and weight_mask: a
 * weight is a nonzero mask bit and a sign, the product adds x where the mask is
 * set, negated where the sign is negative).  The same ternary weights as the
 * 2-bit codes, in another layout: row n is cut into chunks of 32 weights; chunk c
 * holds two little-endian 32-bit words, the mask (bit i set when weight 32 c + i
 * is nonzero) then the sign (bit i set when it is -1; clear for zero weights).
 * K % 32 == 0.  Converted from the 2-bit codes: code 0 -> -1, 1 -> 0, 2 -> +1;
 * a code 3 (which the packer never writes) becomes +1, the nearest value the
 * planes can hold. */
void oracle_pack_bitplanes(const uint8_t *packed, int64_t N, int64_t K, uint8_t *planes) {
    const int64_t KB = K / 4, C = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < C; ++c) {
            uint32_t mask = 0, sign = 0;
            for (int i = 0; i < 32; ++i) {
                const int t = weight_at(packed, KB, n, 32 * c + i);
                if (t != 0) mask |= 1u << i;
                if (t < 0) sign |= 1u << i;
            }
            uint8_t *out = planes + (n * C + c) * 8;
            for (int b = 0; b < 4; ++b) {
                out[b] = (uint8_t)(mask >> (8 * b));
                out[4 + b] = (uint8_t)(sign >> (8 * b));
            }
        }
    }
}

static int bitplane_at(const uint8_t *planes, int64_t K, int64_t n, int64_t k) {
    const uint8_t *ch = planes + (n * (K / 32) + k / 32) * 8;
    const int i = (int)(k % 32);
    const int m = (ch[i / 8] >> (i % 8)) & 1, sg = (ch[4 + i / 8] >> (i % 8)) & 1;
    return m ? (sg ? -1 : 1) : 0;
}

/* acc = sum_k q t over the bitplane weights (exact); y as oracle_linear. */
void oracle_linear_bitplanes(const int8_t *q, const float *s_x, const uint8_t *planes, float s_w, int64_t M,
                             int64_t N, int64_t K, int32_t *acc, float *y) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t a = 0;
            for (int64_t k = 0; k < K; ++k) a += (int64_t)q[m * K + k] * bitplane_at(planes, K, n, k);
            if (acc) acc[m * N + n] = (int32_t)a;
            y[m * N + n] = (float)((double)a * row_factor(s_x[m], s_w));
        }
    }
}

/* --- bf16 output ---------------------------------------------------------- */

/* Each finite fp32 value rounded to the nearest bfloat16 (8 significand bits,
 * the exponent range of fp32), ties to the even significand: IEEE 754
 * round-to-nearest-even into that format.  Written from the definition: the
 * two bf16 neighbours of |f| are its truncation `lo` and lo plus one unit in
 * its last place; the nearer one wins, a tie goes to the one whose last
 * significand bit is 0.  Above the largest finite bf16 the upper neighbour is
 * 2^128, i.e. the result is infinity, as IEEE overflow under this rounding. */
void oracle_to_bf16(const float *y, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &y[i], sizeof u);
        const uint16_t lo = (uint16_t)(u >> 16);          /* sign kept, |value| <= |f| */
        const double a = fabs((double)y[i]);
        const double a_lo = fabs((double)bf16_to_float(lo));
        if (a == a_lo) { out[i] = lo; continue; }
        const int e = (lo >> 7) & 0xFF;                    /* biased exponent of lo */
        const double ulp = ldexp(1.0, (e == 0 ? 1 : e) - 127 - 7);
        const double d_lo = a - a_lo, d_hi = (a_lo + ulp) - a;   /* both exact in float64 */
        if (d_lo < d_hi || (d_lo == d_hi && (lo & 1) == 0)) out[i] = lo;
        else out[i] = (uint16_t)(lo + 1);
    }
}
