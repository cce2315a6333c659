// Per-token absmax int8 activation quantization (page chenxutan.com, sec. 2.2,
// absmax_quantize with 8 bits: qmax = 127).
//
// One workgroup per row: pass 1 takes max|x| over the row (an integer max of the
// bf16 magnitude bits, exact and order-free; wavefront shuffles, then LDS across
// the 4 waves), pass 2 re-reads the row (L2-resident) and writes
// q = rint((127 * x) / s) as int8, 8 codes per 8-byte store.  127 * x is exact
// in binary32 for bf16 x and the quotient is the correctly rounded IEEE one (the
// vector path multiplies by 1 / s and divides only near a rounding boundary).
#include "device_common.h"
#include "internal.h"

namespace bitnet {

constexpr int kQThreads = 256;

template <bool VEC>
__device__ __forceinline__ void quant_row(const uint16_t *__restrict__ x, int K,
                                          int8_t *__restrict__ q, float *__restrict__ s_out) {
    __shared__ uint32_t red[kQThreads / 64];
    const int tid = threadIdx.x;
    uint32_t mx = 0;
    // VEC: the first kHold pieces of 8 values of each thread stay in registers from the
    // max to the codes (all of K <= 8192); later pieces are read again
    constexpr int kHold = 4;
    uint4 held[kHold];
    if (VEC) {
        const uint4 *xv = reinterpret_cast<const uint4 *>(x);
        #pragma unroll
        for (int j = 0; j < kHold; ++j) {
            const int v = tid + kQThreads * j;
            held[j] = v < (K >> 3) ? xv[v] : make_uint4(0u, 0u, 0u, 0u);
            mx = max(mx, absmax8(held[j]));
        }
        for (int v = tid + kQThreads * kHold; v < (K >> 3); v += kQThreads) mx = max(mx, absmax8(xv[v]));
    } else {
        for (int k = tid; k < K; k += kQThreads) mx = max(mx, (uint32_t)(x[k] & 0x7FFFu));
    }
    mx = wave_max_u32(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const float s = bf16f(mx);
    const float inv = 1.0f / s;
    if (tid == 0) *s_out = s;
    if (VEC) {
        const uint4 *xv = reinterpret_cast<const uint4 *>(x);
        uint2 *qv = reinterpret_cast<uint2 *>(q);
        #pragma unroll
        for (int j = 0; j < kHold; ++j) {
            const int v = tid + kQThreads * j;
            if (v < (K >> 3)) qv[v] = mx != 0 ? qcode8(held[j], s, inv) : make_uint2(0u, 0u);
        }
        for (int v = tid + kQThreads * kHold; v < (K >> 3); v += kQThreads) {
            qv[v] = mx != 0 ? qcode8(xv[v], s, inv) : make_uint2(0u, 0u);
        }
    } else {
        for (int k = tid; k < K; k += kQThreads)
            q[k] = (mx != 0) ? (int8_t)qcode(bf16f(x[k]), s) : (int8_t)0;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(const uint16_t *__restrict__ x, int K,
                                                              int8_t *__restrict__ q,
                                                              float *__restrict__ s_x) {
    const size_t m = blockIdx.x;
    quant_row<VEC>(x + m * K, K, q + m * K, s_x + m);
}

__global__ __launch_bounds__(kQThreads) void quant_act_grouped_kernel(const uint8_t *__restrict__ plan) {
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[blockIdx.x];
    const QuantDescDev d = reinterpret_cast<const QuantDescDev *>(plan + h->desc_offset)[e.desc];
    const size_t m = e.local;
    quant_row<true>(d.x + m * d.K, d.K, d.q + m * d.K, d.s_x + m);
}

// RMSNorm of the row with gain g, then the same quantization of the normalized row
// (device_common.h, rms_*): pass 1 takes max|x g| (float64, exact) and sum x^2
// (float64), reduced over the workgroup; pass 2 re-reads the row and writes the codes.
// Vector path: K % 8 == 0, x and q 16-byte aligned, g 16-byte aligned.
__global__ __launch_bounds__(kQThreads) void rmsnorm_quant_kernel(const uint16_t *__restrict__ x,
                                                                  const float *__restrict__ g, float eps,
                                                                  int K, int8_t *__restrict__ q,
                                                                  float *__restrict__ s_x) {
    __shared__ double red[2][kQThreads / 64];
    const size_t m = blockIdx.x;
    const uint16_t *xr = x + m * K;
    int8_t *qr = q + m * K;
    const int tid = threadIdx.x;
    const uint4 *xv = reinterpret_cast<const uint4 *>(xr);
    const float4 *gv = reinterpret_cast<const float4 *>(g);
    double mz = 0.0, ss = 0.0;
    for (int v = tid; v < (K >> 3); v += kQThreads) rms_acc8(xv[v], gv[2 * v], gv[2 * v + 1], mz, ss);
    mz = wave_max_f64(mz);
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) { red[0][tid >> 6] = mz; red[1][tid >> 6] = ss; }
    __syncthreads();
    mz = red[0][0];
    ss = red[1][0];
    #pragma unroll
    for (int w = 1; w < kQThreads / 64; ++w) { mz = fmax(mz, red[0][w]); ss += red[1][w]; }
    if (tid == 0) s_x[m] = rms_scale(mz, ss, K, eps);
    const double c = mz > 0.0 ? 127.0 / mz : 0.0;
    uint2 *qv = reinterpret_cast<uint2 *>(qr);
    for (int v = tid; v < (K >> 3); v += kQThreads)
        qv[v] = mz > 0.0 ? rms_code8(xv[v], gv[2 * v], gv[2 * v + 1], c, mz) : make_uint2(0u, 0u);
}

// SwiGLU of the fp32 gate and up rows, then the quantization of the result
// (device_common.h, swiglu_*): pass 1 forms a and takes max|a| (an integer max of
// the magnitude bits, exact and order-free), pass 2 writes the codes.  The values a
// of each thread's first kHold vectors of 8 stay in registers between the passes;
// later vectors (K > 8 kQThreads kHold) are formed again.  K % 8 == 0; g, u and q
// 16-byte aligned.
__global__ __launch_bounds__(kQThreads) void swiglu_quant_kernel(const float *__restrict__ g,
                                                                 const float *__restrict__ u, int K,
                                                                 int8_t *__restrict__ q,
                                                                 float *__restrict__ s_x) {
    constexpr int kHold = 4;
    __shared__ uint32_t red[kQThreads / 64];
    const size_t m = blockIdx.x;
    const int tid = threadIdx.x, nv = K >> 3;
    const float4 *gv = reinterpret_cast<const float4 *>(g + m * K);
    const float4 *uv = reinterpret_cast<const float4 *>(u + m * K);
    float a[kHold][8];
    uint32_t mx = 0;
    #pragma unroll
    for (int j = 0; j < kHold; ++j) {
        const int v = tid + kQThreads * j;
        if (v < nv) mx = max(mx, swiglu8(gv[2 * v], gv[2 * v + 1], uv[2 * v], uv[2 * v + 1], a[j]));
    }
    for (int v = tid + kQThreads * kHold; v < nv; v += kQThreads) {
        float t[8];
        mx = max(mx, swiglu8(gv[2 * v], gv[2 * v + 1], uv[2 * v], uv[2 * v + 1], t));
    }
    mx = wave_max_u32(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const float s = __uint_as_float(mx);
    const float inv = 1.0f / s;
    if (tid == 0) s_x[m] = s;
    uint2 *qv = reinterpret_cast<uint2 *>(q + m * K);
    #pragma unroll
    for (int j = 0; j < kHold; ++j) {
        const int v = tid + kQThreads * j;
        if (v < nv) qv[v] = mx != 0 ? qcode8_f32(a[j], s, inv) : make_uint2(0u, 0u);
    }
    for (int v = tid + kQThreads * kHold; v < nv; v += kQThreads) {
        float t[8];
        swiglu8(gv[2 * v], gv[2 * v + 1], uv[2 * v], uv[2 * v + 1], t);
        qv[v] = mx != 0 ? qcode8_f32(t, s, inv) : make_uint2(0u, 0u);
    }
}

hipError_t launch_swiglu_quant(const float *g, const float *u, int64_t M, int64_t K, int8_t *q, float *s_x,
                               hipStream_t st) {
    swiglu_quant_kernel<<<dim3((unsigned)M), dim3(kQThreads), 0, st>>>(g, u, (int)K, q, s_x);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_quant(const uint16_t *x, const float *g, float eps, int64_t M, int64_t K, int8_t *q,
                                float *s_x, hipStream_t st) {
    rmsnorm_quant_kernel<<<dim3((unsigned)M), dim3(kQThreads), 0, st>>>(x, g, eps, (int)K, q, s_x);
    return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s_x,
                            hipStream_t st) {
    const bool vec = (K % 8 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)q % 16 == 0);
    dim3 grid((unsigned)M), block(kQThreads);
    if (vec)
        quant_act_kernel<true><<<grid, block, 0, st>>>(x, (int)K, q, s_x);
    else
        quant_act_kernel<false><<<grid, block, 0, st>>>(x, (int)K, q, s_x);
    return hipGetLastError();
}

hipError_t launch_quant_act_grouped(const void *plan_dev, uint32_t blocks, hipStream_t st) {
    quant_act_grouped_kernel<<<dim3(blocks), dim3(kQThreads), 0, st>>>(
        reinterpret_cast<const uint8_t *>(plan_dev));
    return hipGetLastError();
}

}  // namespace bitnet
