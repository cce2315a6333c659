// Absmean ternarization and 2-bit packing of a weight tensor (pages:
// chenxutan.com sec. 2.2 absmean_quantize and sec. 3.3 pack_ternary;
// 0539edu.com sec. 2.1 RoundClip with scale = mean|w|).  Offline step.
//
//  1. rowsum_kernel   : one thread per row, sum_k |w| in float64 in increasing k
//                       (the order is part of the result, so it is fixed);
//  2. combine_kernel  : one thread, sum_n rowsum in increasing n, one rounding of
//                       the mean to fp32 -> s_w;
//  3. code_kernel     : t = clamp(rint(w / (s_w + eps)), -1, 1) with binary32
//                       ops, code t + 1, four codes per byte, LSB first; works on
//                       the flat array (K % 4 == 0 keeps bytes inside rows).
#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace bitnet {

__global__ __launch_bounds__(64) void rowsum_kernel(const float *__restrict__ w, int64_t N, int64_t K,
                                                    double *__restrict__ rowsum) {
    const int64_t n = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (n >= N) return;
    const float *r = w + n * K;
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += fabs((double)r[k]);
    rowsum[n] = s;
}

__global__ __launch_bounds__(64) void combine_kernel(const double *__restrict__ rowsum, int64_t N,
                                                     int64_t K, float *__restrict__ s_w) {
    if (threadIdx.x != 0) return;
    double t = 0.0;
    for (int64_t n = 0; n < N; ++n) t += rowsum[n];
    *s_w = (N * K == 0) ? 0.0f : (float)(t / (double)(N * K));
}

__device__ __forceinline__ uint32_t code_of(float w, float d) {
    float r = __builtin_rintf(w / d);
    r = fminf(fmaxf(r, -1.0f), 1.0f);
    return (uint32_t)((int)r + 1);
}

__global__ __launch_bounds__(256) void code_kernel(const float *__restrict__ w, int64_t nbytes,
                                                   float eps, const float *__restrict__ s_w,
                                                   uint8_t *__restrict__ packed) {
    const int64_t j4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // first byte of this thread
    if (j4 >= nbytes) return;
    const float d = *s_w + eps;
    const int nb = (int)min((int64_t)4, nbytes - j4);
    uint32_t out = 0;
    for (int b = 0; b < nb; ++b) {
        const float *p = w + (j4 + b) * 4;
        uint32_t byte = code_of(p[0], d) | code_of(p[1], d) << 2 | code_of(p[2], d) << 4 |
                        code_of(p[3], d) << 6;
        out |= byte << (8 * b);
    }
    if (nb == 4 && ((uintptr_t)(packed + j4) % 4 == 0)) {
        *reinterpret_cast<uint32_t *>(packed + j4) = out;
    } else {
        for (int b = 0; b < nb; ++b) packed[j4 + b] = (uint8_t)(out >> (8 * b));
    }
}

// Group-wise scales (pages: chenxutan.com sec. 3.1 weight_scale per output channel,
// sec. 4.3 group-wise quantization; 0539edu.com sec. 2.1 scales per channel): row n
// is cut into K / G groups of G consecutive weights; each gets its own absmean scale
// s = fp32(mean |w|) (float64 sum, k ascending) and its codes rint(w / (s + eps))
// clamped to [-1, 1].  s_w is [N][K / G]; G = K is one scale per output channel.
__global__ __launch_bounds__(64) void group_scale_kernel(const float *__restrict__ w, int64_t N, int64_t K,
                                                         int64_t G, float *__restrict__ s_w) {
    const int64_t ng = K / G;
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;   // (n, g)
    if (i >= N * ng) return;
    const int64_t n = i / ng, g = i - n * ng;
    const float *r = w + n * K + g * G;
    double s = 0.0;
    for (int64_t k = 0; k < G; ++k) s += fabs((double)r[k]);
    s_w[i] = (float)(s / (double)G);
}

__global__ __launch_bounds__(256) void code_grouped_kernel(const float *__restrict__ w, int64_t N, int64_t K,
                                                           int64_t G, float eps, const float *__restrict__ s_w,
                                                           uint8_t *__restrict__ packed) {
    const int64_t KB = K / 4, ng = K / G;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;   // byte index
    if (j >= N * KB) return;
    const int64_t n = j / KB, k = 4 * (j - n * KB);               // G % 4 == 0: one group per byte
    const float d = s_w[n * ng + k / G] + eps;
    const float *p = w + n * K + k;
    packed[j] = (uint8_t)(code_of(p[0], d) | code_of(p[1], d) << 2 | code_of(p[2], d) << 4 | code_of(p[3], d) << 6);
}

hipError_t launch_pack_grouped(const float *w, int64_t N, int64_t K, int64_t G, float eps, uint8_t *packed,
                               float *s_w, hipStream_t st) {
    const int64_t pairs = N * (K / G);
    group_scale_kernel<<<dim3((unsigned)((pairs + 63) / 64)), dim3(64), 0, st>>>(w, N, K, G, s_w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nbytes = N * K / 4;
    code_grouped_kernel<<<dim3((unsigned)((nbytes + 255) / 256)), dim3(256), 0, st>>>(w, N, K, G, eps, s_w, packed);
    return hipGetLastError();
}

hipError_t launch_weight_scale(const float *w, int64_t N, int64_t K, float *s_w, double *rowsum, hipStream_t st) {
    if (N > 0) {
        rowsum_kernel<<<dim3((unsigned)((N + 63) / 64)), dim3(64), 0, st>>>(w, N, K, rowsum);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    combine_kernel<<<dim3(1), dim3(64), 0, st>>>(rowsum, N, K, s_w);
    return hipGetLastError();
}

// Scratch for callers that cannot allocate: the float64 row sums of one pack call
// live in this array instead of a caller workspace.  Each GPU holds its own copy
// for the life of the process; host code must use the address hipGetSymbolAddress
// reports for the current device (the array's name on the host is only a stand-in,
// and a kernel handed it would fault).
static __device__ __align__(256) double scratch[kPackScratchRows];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices] = {};
}  // namespace

hipError_t pack_scratch(double **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = p;
    }
    *out = static_cast<double *>(g_scratch_dev[dev]);
    return hipSuccess;
}

hipError_t launch_pack(const float *w, int64_t N, int64_t K, float eps, uint8_t *packed, float *s_w,
                       double *rowsum, hipStream_t st) {
    hipError_t e = launch_weight_scale(w, N, K, s_w, rowsum, st);
    if (e != hipSuccess || N == 0) return e;
    const int64_t nbytes = N * K / 4;
    const int64_t threads = (nbytes + 3) / 4;
    code_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st>>>(w, nbytes, eps, s_w,
                                                                               packed);
    return hipGetLastError();
}

}  // namespace bitnet
