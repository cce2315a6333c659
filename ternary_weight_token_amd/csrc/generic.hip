// General contraction kernel for shapes the fast kernels do not take
// (K % 64 != 0 or unaligned q / packed): one thread per output, byte loads.
// Same definition and results as the fast kernels (pages: chenxutan.com
// sec. 2.3 and sec. 3.1).
#include "device_common.h"
#include "internal.h"

namespace bitnet {

__global__ __launch_bounds__(256) void linear_generic_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s_x, const uint8_t *__restrict__ packed,
    const float *__restrict__ s_w, int64_t M, int64_t N, int64_t K, const OutSpec out,
    int32_t *__restrict__ acc_out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx % N;
    const int8_t *qr = q + m * K;
    const uint8_t *pr = packed + n * (K / 4);
    if (out.w_group == 0) {
        int s = 0;
        for (int64_t j = 0; j < K / 4; ++j) {
            const uint32_t b = pr[j];
            #pragma unroll
            for (int i = 0; i < 4; ++i) s += (int)qr[4 * j + i] * ((int)((b >> (2 * i)) & 3u) - 1);
        }
        put_y(out, idx, (int)n, s, rescale_factor(s_x[m], *s_w));
        if (acc_out) acc_out[idx] = s;
        return;
    }
    // weight scales per group of G = w_group weights of the row: y = fp32((sum_g
    // acc_g s_w[n][g]) s_x / 127), the sum in float64; G = K (one scale per output
    // channel) is the per-tensor rescale with the row's own scale
    const int64_t G = out.w_group, ng = K / G;
    int total = 0;
    double v = 0.0;
    for (int64_t g = 0; g < ng; ++g) {
        int a = 0;
        for (int64_t j = g * G / 4; j < (g + 1) * G / 4; ++j) {
            const uint32_t b = pr[j];
            #pragma unroll
            for (int i = 0; i < 4; ++i) a += (int)qr[4 * j + i] * ((int)((b >> (2 * i)) & 3u) - 1);
        }
        total += a;
        v += (double)a * (double)s_w[n * ng + g];
    }
    if (ng == 1) v = (double)total * rescale_factor(s_x[m], s_w[n]);
    else v = (v * (double)s_x[m]) / 127.0;
    if (out.bias) v += (double)out.bias[n];
    store_y(out, idx, v);
    if (acc_out) acc_out[idx] = total;
}

hipError_t launch_linear_generic(const int8_t *q, const float *s_x, const uint8_t *packed,
                                 const float *s_w, int64_t M, int64_t N, int64_t K, const OutSpec &y,
                                 int32_t *acc, hipStream_t st) {
    const int64_t total = M * N;
    linear_generic_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st>>>(
        q, s_x, packed, s_w, M, N, K, y, acc);
    return hipGetLastError();
}

}  // namespace bitnet
