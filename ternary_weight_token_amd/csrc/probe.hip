// Measurement probes: a streaming read of a device buffer and a loop of int8
// MFMAs on registers, the achievable ceilings of the HBM stream and of the int8
// matrix cores next to which the BitLinear kernels are measured.
#include "device_common.h"
#include "internal.h"

namespace bitnet {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;      // 16-byte loads in flight per thread
constexpr int kProbeChains = 8;      // independent MFMA accumulators per wavefront
// 8 wavefronts per workgroup: at this size the compiler keeps the accumulators in
// place (with 4, it rotates them through accumulation registers every round)
constexpr int kProbeMfmaThreads = 512;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint8_t *__restrict__ buf, int64_t chunks,
                                                                   uint32_t key, uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t fold = 0;
    // whole rounds: kProbeUnroll loads per thread, each one lane-linear across the grid
    for (; i + (kProbeUnroll - 1) * stride < chunks; i += kProbeUnroll * stride) {
        v4u v[kProbeUnroll];
        #pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load((gv4u *)(buf + 16 * (i + u * stride)));
        #pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < chunks; i += stride) {
        const v4u v = __builtin_nontemporal_load((gv4u *)(buf + 16 * i));
        fold ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (fold == key) sink[0] = fold;
}

typedef int pv4i __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeMfmaThreads) void mfma_i8_kernel(int iters, uint32_t key, uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const pv4i a{(int)(key ^ lane), (int)(key * 3u), (int)(key + 7u * lane), (int)~key};
    const pv4i b{(int)(key >> 3), (int)(key ^ 0x5A5A5A5Au), (int)(lane * 0x01010101u), (int)(key + 1u)};
    pv4i acc[kProbeChains];
    #pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = pv4i{c, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        #pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
    }
    uint32_t fold = 0;
    #pragma unroll
    for (int c = 0; c < kProbeChains; ++c) fold ^= (uint32_t)(acc[c].x ^ acc[c].y ^ acc[c].z ^ acc[c].w);
    if (fold == key) sink[0] = fold;
}

}  // namespace

hipError_t launch_probe_stream_read(const void *buf, int64_t bytes, int64_t blocks, uint32_t key, uint32_t *sink,
                                    hipStream_t st) {
    stream_read_kernel<<<dim3((unsigned)blocks), dim3(kProbeThreads), 0, st>>>(
        static_cast<const uint8_t *>(buf), bytes / 16, key, sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma_i8(int64_t blocks, int64_t iters, uint32_t key, uint32_t *sink, hipStream_t st) {
    mfma_i8_kernel<<<dim3((unsigned)blocks), dim3(kProbeMfmaThreads), 0, st>>>((int)iters, key, sink);
    return hipGetLastError();
}

double probe_mfma_i8_ops(int64_t blocks, int64_t iters) {
    // 8 wavefronts x chains x iters MFMAs of 16 x 16 x 64 multiply-adds
    return (double)blocks * (kProbeMfmaThreads / 64) * kProbeChains * (double)iters * (2.0 * 16 * 16 * 64);
}

}  // namespace bitnet
