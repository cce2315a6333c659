// Decode GEMV (M <= 16): acc[m][n] = sum_k q[m][k] * t[n][k], y = acc * s_x * s_w / 127
// (pages: chenxutan.com sec. 2.3 rescale and sec. 3.1 BitLinear.forward; the
// ternary product is an add / subtract / skip, chenxutan.com sec. 1).
//
// HBM-bound: every packed weight byte is read exactly once.  Layout of the work:
//  * a wavefront owns RG row groups of 8 rows; the 8 lanes of an octet walk one
//    row, lane l8 taking 16-byte chunks l8, l8 + 8, ... (one chunk = 64 weights),
//    so one load instruction reads 8 rows x 128 contiguous bytes;
//  * the 2-bit codes c = t + 1 are regrouped in registers with shift+mask
//    (codes_i) and fed to v_dot4_i32_i8 unshifted; sum_k q * t is then
//    sum_k q * c - sum_k q, the second term costing 16 dot4 per chunk and row of q
//    instead of one subtraction per weight;
//  * the 64 q bytes of a chunk are loaded once per chunk (L2/L1-resident) and
//    byte-transposed to the order codes_i produces; they are reused by every row
//    group of the wavefront;
//  * partial sums are reduced across the octet with DPP; when the workgroup has
//    several wavefronts they split K and combine their partials through LDS;
//  * epilogue: y = fp32(acc * c_m), c_m = (s_x[m] * s_w) / 127 in float64.
#include "device_common.h"
#include "internal.h"

namespace bitnet {

constexpr int kMaxKSplit = 8;

template <int MT, int RG>
__device__ __forceinline__ void gemv_tile(const int8_t *__restrict__ q, const float *__restrict__ s_x,
                                          const uint8_t *__restrict__ packed,
                                          const float *__restrict__ s_w, int M, int N, int K,
                                          float *__restrict__ y, int32_t *__restrict__ acc_out,
                                          int row0, int m0, int kslices, int *lds) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l8 = lane & 7;
    const int rs = lane >> 3;
    const int C = K >> 6;     // 16-byte chunks per packed row
    const int KB = K >> 2;    // bytes per packed row
    const int cb = (int)(((int64_t)C * wave) / kslices);
    const int ce = (int)(((int64_t)C * (wave + 1)) / kslices);
    const int mcount = min(MT, M - m0);

    int acc[RG][MT];
    const uint8_t *prow[RG];
    #pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int r = row0 + 8 * g + rs;
        prow[g] = packed + (size_t)(r < N ? r : 0) * KB;   // rows past N read row 0, discarded
        #pragma unroll
        for (int m = 0; m < MT; ++m) acc[g][m] = 0;
    }
    const int8_t *qrow = q + (size_t)m0 * K;

    for (int c = cb + l8; c < ce; c += 8) {
        uint4 wv[RG];
        #pragma unroll
        for (int g = 0; g < RG; ++g) wv[g] = *reinterpret_cast<const uint4 *>(prow[g] + 16 * c);
        #pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mcount) {
                const uint4 *qp = reinterpret_cast<const uint4 *>(qrow + (size_t)m * K + 64 * c);
                uint4 a[4] = {qp[0], qp[1], qp[2], qp[3]};
                uint32_t P[4][4];
                int sq = 0;
                #pragma unroll
                for (int d = 0; d < 4; ++d) {
                    transpose4x4(a[d].x, a[d].y, a[d].z, a[d].w, P[d][0], P[d][1], P[d][2], P[d][3]);
                    sq = dot4(a[d].x, 0x01010101u, sq);
                    sq = dot4(a[d].y, 0x01010101u, sq);
                    sq = dot4(a[d].z, 0x01010101u, sq);
                    sq = dot4(a[d].w, 0x01010101u, sq);
                }
                #pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const uint32_t wd[4] = {wv[g].x, wv[g].y, wv[g].z, wv[g].w};
                    int s = acc[g][m] - sq;
                    #pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        #pragma unroll
                        for (int i = 0; i < 4; ++i) s = dot4(codes_i(wd[d], i), P[d][i], s);
                    }
                    acc[g][m] = s;
                }
            }
        }
    }

    #pragma unroll
    for (int g = 0; g < RG; ++g) {
        #pragma unroll
        for (int m = 0; m < MT; ++m) acc[g][m] = octet_sum(acc[g][m]);
    }

    const float sw = *s_w;
    if (kslices == 1) {
        #pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int r = row0 + 8 * g + rs;
            if (r >= N) continue;
            #pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mcount && l8 == (m & 7)) {
                    const size_t o = (size_t)(m0 + m) * N + r;
                    y[o] = rescale(acc[g][m], rescale_factor(s_x[m0 + m], sw));
                    if (acc_out) acc_out[o] = acc[g][m];
                }
            }
        }
        return;
    }
    // K split across the workgroup's wavefronts: combine through LDS.
    constexpr int R = 8 * RG;
    if (l8 == 0) {
        #pragma unroll
        for (int g = 0; g < RG; ++g) {
            #pragma unroll
            for (int m = 0; m < MT; ++m) lds[(wave * R + 8 * g + rs) * MT + m] = acc[g][m];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < R * MT; idx += blockDim.x) {
        const int rr = idx / MT, m = idx % MT;
        const int r = row0 + rr;
        if (r >= N || m >= mcount) continue;
        int s = 0;
        for (int w = 0; w < kslices; ++w) s += lds[(w * R + rr) * MT + m];
        const size_t o = (size_t)(m0 + m) * N + r;
        y[o] = rescale(s, rescale_factor(s_x[m0 + m], sw));
        if (acc_out) acc_out[o] = s;
    }
}

template <int MT, int RG>
__global__ __launch_bounds__(64 * kMaxKSplit) void gemv_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s_x, const uint8_t *__restrict__ packed,
    const float *__restrict__ s_w, int M, int N, int K, float *__restrict__ y,
    int32_t *__restrict__ acc_out, int kslices) {
    __shared__ int lds[kMaxKSplit * 8 * RG * MT];
    gemv_tile<MT, RG>(q, s_x, packed, s_w, M, N, K, y, acc_out, blockIdx.x * 8 * RG, blockIdx.y * MT,
                      kslices, lds);
}

// Grouped decode: one wavefront per block, block -> (descriptor, row set, M tile)
// through the plan's block table.
constexpr int kGroupedRG = 4;
constexpr int kGroupedMT = 1;

__global__ __launch_bounds__(64) void gemv_grouped_kernel(const uint8_t *__restrict__ plan) {
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[blockIdx.x];
    const LinearDescDev d = reinterpret_cast<const LinearDescDev *>(plan + h->desc_offset)[e.desc];
    const int rowsets = (d.N + 8 * kGroupedRG - 1) / (8 * kGroupedRG);
    const int rs = (int)(e.local % rowsets), mt = (int)(e.local / rowsets);
    gemv_tile<kGroupedMT, kGroupedRG>(d.q, d.s_x, d.packed, d.s_w, d.M, d.N, d.K, d.y, d.acc,
                                      rs * 8 * kGroupedRG, mt * kGroupedMT, 1, nullptr);
}

uint32_t gemv_grouped_rows_per_block() { return 8 * kGroupedRG; }
uint32_t gemv_grouped_threads() { return 64; }
uint32_t gemv_grouped_mtile() { return kGroupedMT; }

template <int MT, int RG>
static hipError_t launch_t(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                           int64_t M, int64_t N, int64_t K, float *y, int32_t *acc, hipStream_t st) {
    const int rows = 8 * RG;
    const unsigned gx = (unsigned)((N + rows - 1) / rows);
    const unsigned gy = (unsigned)((M + MT - 1) / MT);
    const int C = (int)(K / 64);
    // split K across wavefronts until the launch has ~8 wavefronts per CU, keeping
    // at least 4 chunk iterations per lane.
    int ks = 1;
    while (ks < kMaxKSplit && (int64_t)gx * gy * ks < 2048 && C / (16 * ks) >= 4) ks *= 2;
    gemv_kernel<MT, RG><<<dim3(gx, gy), dim3(64 * ks), 0, st>>>(q, s_x, packed, s_w, (int)M, (int)N,
                                                                (int)K, y, acc, ks);
    return hipGetLastError();
}

hipError_t launch_gemv(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                       int64_t M, int64_t N, int64_t K, float *y, int32_t *acc, hipStream_t st) {
    if (M == 1) return launch_t<1, 4>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    if (M == 2) return launch_t<2, 4>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    if (M <= 4) return launch_t<4, 2>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    return launch_t<8, 2>(q, s_x, packed, s_w, M, N, K, y, acc, st);
}

hipError_t launch_gemv_grouped(const void *plan_dev, uint32_t blocks, hipStream_t st) {
    gemv_grouped_kernel<<<dim3(blocks), dim3(64), 0, st>>>(reinterpret_cast<const uint8_t *>(plan_dev));
    return hipGetLastError();
}

}  // namespace bitnet
