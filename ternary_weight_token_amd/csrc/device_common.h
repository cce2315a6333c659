// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace bitnet {

// Global loads go through the global address space explicitly: pointers read
// from a plan descriptor are otherwise generic (FLAT) accesses, which also count
// against the LDS wait counter and would serialise them with the LDS reads.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u gv4u;

__device__ __forceinline__ uint4 gload16(const void *p) {
    const v4u v = *(gv4u *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Weight loads: nontemporal when NT (each packed byte is read once per launch).
template <bool NT>
__device__ __forceinline__ uint4 load_weights(const uint8_t *p) {
    if (NT) {
        const v4u v = __builtin_nontemporal_load((gv4u *)p);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return gload16(p);
}

// Four signed bytes of `a` dotted with four signed bytes of `b`, plus c
// (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Codes of one packed dword (16 weights: byte b holds k = 4b + i in bits 2i..2i+1)
// regrouped by i: lane i of the result holds, in byte b, the code of k = 4b + i.
__device__ __forceinline__ uint32_t codes_i(uint32_t w, int i) {
    return (w >> (2 * i)) & 0x03030303u;
}

// Ternary value (code - 1) of four codes held one per byte: v_perm_b32 used as
// a 4-entry byte table {0xFF, 0x00, 0x01, 0x02}.
__device__ __forceinline__ uint32_t codes_to_ternary(uint32_t c) {
    return __builtin_amdgcn_perm(0u, 0x020100FFu, c);
}

// 4x4 byte transpose: given natural dwords Q0..Q3 (Qj byte b = element 4j + b)
// return P0..P3 with Pi byte b = element 4b + i, the order codes_i() produces.
__device__ __forceinline__ void transpose4x4(uint32_t q0, uint32_t q1, uint32_t q2, uint32_t q3,
                                             uint32_t &p0, uint32_t &p1, uint32_t &p2, uint32_t &p3) {
    // v_perm_b32(a, b, sel): selector 0..3 picks bytes of b, 4..7 bytes of a.
    uint32_t t0 = __builtin_amdgcn_perm(q1, q0, 0x05010400u);  // q0.b0 q1.b0 q0.b1 q1.b1
    uint32_t t1 = __builtin_amdgcn_perm(q3, q2, 0x05010400u);  // q2.b0 q3.b0 q2.b1 q3.b1
    uint32_t t2 = __builtin_amdgcn_perm(q1, q0, 0x07030602u);  // q0.b2 q1.b2 q0.b3 q1.b3
    uint32_t t3 = __builtin_amdgcn_perm(q3, q2, 0x07030602u);  // q2.b2 q3.b2 q2.b3 q3.b3
    p0 = __builtin_amdgcn_perm(t1, t0, 0x05040100u);           // q0.b0 q1.b0 q2.b0 q3.b0
    p1 = __builtin_amdgcn_perm(t1, t0, 0x07060302u);           // q0.b1 q1.b1 q2.b1 q3.b1
    p2 = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
    p3 = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
}

// Eight unsigned / signed 4-bit products summed, plus c (v_dot8_u32_u4 /
// v_dot8_i32_i4).
__device__ __forceinline__ uint32_t udot8(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_udot8(a, b, c, false);
}
__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}

// Nibble form of 16 int8 activations q_0..q_15 (natural dwords Q0..Q3, Qj byte b
// = q_{4j+b}) for a product with the 16 two-bit codes of one packed dword.
// Write q = 16 h + l with l = q & 15 (unsigned) and h = q >> 4 (signed 4-bit).
// Codes split as u0 = w & 0x33333333 (nibble j = code of element 2j) and
// u1 = (w >> 2) & 0x33333333 (nibble j = code of element 2j + 1); the matching
// activation nibbles are
//   le / he : nibble j = l_{2j} / h_{2j},   lo / ho : nibble j = l_{2j+1} / h_{2j+1}
// so that  sum_k q_k c_k = 16 (sdot8(u0, he) + sdot8(u1, ho)) + udot8(u0, le) + udot8(u1, lo).
struct QNib { uint32_t le, he, lo, ho; };

__device__ __forceinline__ QNib nibble_form(uint32_t q0, uint32_t q1, uint32_t q2, uint32_t q3) {
    uint32_t p0, p1, p2, p3;  // p_i byte b = q_{4b+i}
    transpose4x4(q0, q1, q2, q3, p0, p1, p2, p3);
    const uint32_t m = 0x0F0F0F0Fu;
    QNib r;
    r.le = (p0 & m) | ((p2 << 4) & ~m);   // byte b: l_{4b} | l_{4b+2} << 4
    r.he = ((p0 >> 4) & m) | (p2 & ~m);   // byte b: h_{4b} | h_{4b+2} << 4
    r.lo = (p1 & m) | ((p3 << 4) & ~m);
    r.ho = ((p1 >> 4) & m) | (p3 & ~m);
    return r;
}

// Sum over the 8 lanes of each aligned lane octet (DPP: quad swaps, then the
// half-row mirror, which pairs lane i with lane 7 - i of the octet).
__device__ __forceinline__ int octet_sum(int v) {
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);  // row_half_mirror
    return v;
}

// Sum over the 8 lanes of an octet, float64 (shuffles within the octet).
__device__ __forceinline__ double octet_sum_f64(double v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    return v;
}

// Full-wavefront max of non-negative ints (64 lanes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    #pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint32_t u = (uint32_t)__shfl_xor((int)v, o, 64);
        v = u > v ? u : v;
    }
    return v;
}

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

// Activation code of x for the row scale s = max|x| > 0 (page chenxutan.com sec. 2.2,
// absmax_quantize, 8 bits): rint((127 x) / s) clamped to [-127, 127].  127 x is exact
// in binary32 for bf16 x and the division is the correctly rounded IEEE one.
__device__ __forceinline__ int qcode(float x, float s) {
    float v = (127.0f * x) / s;
    float r = __builtin_rintf(v);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Largest bf16 magnitude bits (|x| with the sign cleared) among the 8 values of a
// 16-byte vector: an integer max, exact and order-free.
__device__ __forceinline__ uint32_t absmax8(uint4 u) {
    const uint32_t a = max(u.x & 0x7FFFu, u.x >> 16 & 0x7FFFu);
    const uint32_t b = max(u.y & 0x7FFFu, u.y >> 16 & 0x7FFFu);
    const uint32_t c = max(u.z & 0x7FFFu, u.z >> 16 & 0x7FFFu);
    const uint32_t d = max(u.w & 0x7FFFu, u.w >> 16 & 0x7FFFu);
    return max(max(a, b), max(c, d));
}

// The same code with inv = 1 / s (correctly rounded) computed once per row: the
// product (127 x) * inv lies within 1.6e-5 of the exact quotient (|quotient| <= 127,
// two roundings of 2^-24 relative each), so its nearest integer is the exact one
// whenever it is at least 4e-5 away from a half-integer -- and then the binary32
// quotient, within 4e-6 of the exact one, rounds to that integer too.  Otherwise
// (about one code in a thousand, and never for an overflowing or non-finite
// product) the correctly rounded division decides.  An exhaustive test over all
// bf16 inputs checks the result against the plain definition.
__device__ __forceinline__ int qcode_inv(float x, float s, float inv) {
    const float a = 127.0f * x;
    const float t = a * inv;
    float r = __builtin_rintf(t);
    if (!(fabsf(t - r) < 0.49996f)) r = __builtin_rintf(a / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Codes of 8 bf16 values (one 16-byte vector) packed into 8 bytes; inv = 1 / s.
__device__ __forceinline__ uint2 qcode8(uint4 u, float s, float inv) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t b[8];
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        b[2 * j] = (uint32_t)qcode_inv(bf16f(w[j] & 0xFFFFu), s, inv) & 0xFFu;
        b[2 * j + 1] = (uint32_t)qcode_inv(bf16f(w[j] >> 16), s, inv) & 0xFFu;
    }
    return make_uint2(b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24, b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24);
}

// ---- RMSNorm before the quantization (page chenxutan.com sec. 3.1: the block
// normalizes the token row in full precision; the linear layer quantizes the
// result, sec. 2.2).  The normalized value is the real x g r, r = 1 / sqrt(mean(x^2)
// + eps); its absmax codes are rint(127 z / max|z|) with z = x g (r cancels) and
// its scale is max|z| r.  z is exact in float64 (bf16 x, fp32 g), and so is 127 z.

__device__ __forceinline__ double wave_max_f64(double v) {
    #pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    #pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Code of z for mz = max|z| > 0, with c = 127 / mz: t = z c is within 2^-51 |t| of
// 127 z / mz, and a ratio of that form is either exactly a half-integer or at least
// 2^-41 relatively away from one, so rint(t) is the exact rounding unless t lies
// within 2^-45 |t| of a half-integer; there the correctly rounded division decides
// (it keeps an exact tie exact).
__device__ __forceinline__ int rms_code(double z, double c, double mz) {
    const double t = z * c;
    double r = rint(t);
    if (fabs(fabs(t - r) - 0.5) <= 0x1p-45 * fabs(t)) r = rint((127.0 * z) / mz);
    r = fmin(fmax(r, -127.0), 127.0);
    return (int)r;
}

// Codes of 8 values (bf16 x in u, fp32 gains in g0 / g1) as 8 int8 bytes.
__device__ __forceinline__ uint2 rms_code8(uint4 u, float4 g0, float4 g1, double c, double mz) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    uint32_t b[8];
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        b[2 * j] = (uint32_t)rms_code((double)bf16f(w[j] & 0xFFFFu) * (double)g[2 * j], c, mz) & 0xFFu;
        b[2 * j + 1] = (uint32_t)rms_code((double)bf16f(w[j] >> 16) * (double)g[2 * j + 1], c, mz) & 0xFFu;
    }
    return make_uint2(b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24, b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24);
}

// max|x g| and sum x^2 over 8 values.
__device__ __forceinline__ void rms_acc8(uint4 u, float4 g0, float4 g1, double &mz, double &ss) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float xf = bf16f(j & 1 ? w[j >> 1] >> 16 : w[j >> 1] & 0xFFFFu);
        mz = fmax(mz, fabs((double)xf * (double)g[j]));
        ss += (double)(xf * xf);   // x^2 is exact in fp32 for bf16 x
    }
}

// Scale of the normalized row: max|z| / sqrt(mean(x^2) + eps), in float64.
__device__ __forceinline__ float rms_scale(double mz, double ss, int K, float eps) {
    if (mz == 0.0) return 0.0f;
    const double r = 1.0 / sqrt(ss / (double)K + (double)eps);
    return (float)(mz * r);
}

// ---- SwiGLU before the down projection (page chenxutan.com sec. 3.1: the block
// feeds its down projection with silu(gate(h)) * up(h), g and u the fp32 outputs of
// gate and up).  a = g u / (1 + e^-g) is evaluated in float64 and rounded once to
// fp32; the row is then quantized like any other fp32 row (scale max|a|, codes
// rint(127 a / max|a|), qcode_f32).
__device__ __forceinline__ float swiglu_value(float g, float u) {
    const double gd = (double)g;
    return (float)((gd / (1.0 + exp(-gd))) * (double)u);
}

// a of 8 values (g and u as two float4 each); returns the largest |a| bits (|a| as
// an unsigned integer orders like |a| for finite values).
__device__ __forceinline__ uint32_t swiglu8(float4 g0, float4 g1, float4 u0, float4 u1, float (&a)[8]) {
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    uint32_t mx = 0;
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = swiglu_value(g[j], u[j]);
        mx = max(mx, __float_as_uint(a[j]) & 0x7FFFFFFFu);
    }
    return mx;
}

// Code of an fp32 value x for the row scale s = max|x| > 0, inv = 1 / s (correctly
// rounded): rint(127 x / s) of the real quotient.  t = fl(fl(127 x) inv) is within
// 3.0001 2^-24 |127 x / s| <= 2.3e-5 of the quotient (three roundings; 127 x is exact
// when it is subnormal), so when t is at least 4e-5 inside a half-integer interval
// its nearest integer is the quotient's; otherwise (or for a non-finite t: inv
// overflows for a subnormal s) float64 decides, where 127 x is exact and the
// correctly rounded quotient never meets or crosses a half-integer it is not on.
__device__ __forceinline__ int qcode_f32(float x, float s, float inv) {
    const float t = (127.0f * x) * inv;
    float r = __builtin_rintf(t);
    if (!(fabsf(t - r) < 0.49996f)) r = (float)rint((127.0 * (double)x) / (double)s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Codes of 8 fp32 values as 8 int8 bytes.
__device__ __forceinline__ uint2 qcode8_f32(const float (&a)[8], float s, float inv) {
    uint32_t b[8];
    #pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = (uint32_t)qcode_f32(a[j], s, inv) & 0xFFu;
    return make_uint2(b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24, b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24);
}

// Largest |x| bits among 8 fp32 values (|x| as an unsigned integer orders like |x|).
__device__ __forceinline__ uint32_t absmax8_f32(float4 a, float4 b) {
    const uint32_t m = 0x7FFFFFFFu;
    const uint32_t u0 = max(__float_as_uint(a.x) & m, __float_as_uint(a.y) & m);
    const uint32_t u1 = max(__float_as_uint(a.z) & m, __float_as_uint(a.w) & m);
    const uint32_t u2 = max(__float_as_uint(b.x) & m, __float_as_uint(b.y) & m);
    const uint32_t u3 = max(__float_as_uint(b.z) & m, __float_as_uint(b.w) & m);
    return max(max(u0, u1), max(u2, u3));
}

// y = fp32(acc * c) with c = (s_x * s_w) / 127 formed in float64.
__device__ __forceinline__ double rescale_factor(float s_x, float s_w) {
    return ((double)s_x * (double)s_w) / 127.0;
}
__device__ __forceinline__ float rescale(int acc, double c) {
    return (float)((double)acc * c);
}

// bf16 nearest-even rounding of a finite fp32 value.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Round the float64 output value once to fp32 and store it (as bf16 if asked).
__device__ __forceinline__ void store_y(const OutSpec &out, size_t o, double v) {
    const float f = (float)v;
    if (out.bf16) reinterpret_cast<uint16_t *>(out.y)[o] = bf16_rne(f);
    else reinterpret_cast<float *>(out.y)[o] = f;
}

// Rescale factor of output column n: the per-tensor c_m when the weights have one
// scale, else (s_x[m] * s_w[n]) / 127 with the column's own scale (w_group = K).
__device__ __forceinline__ double col_factor(const OutSpec &out, const float *s_w, int n, float sxm, double cm) {
    return out.w_group ? rescale_factor(sxm, s_w[n]) : cm;
}

// Store output element o (column n) from acc and c = c_m; see OutSpec.
__device__ __forceinline__ void put_y(const OutSpec &out, size_t o, int n, int acc, double c) {
    double v = (double)acc * c;
    if (out.bias) v += (double)out.bias[n];
    store_y(out, o, v);
}

}  // namespace bitnet
