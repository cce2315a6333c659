// Prefill GEMM (M > 16): the same contraction and rescale as the GEMV, as a dense
// int8 x ternary -> int32 product on the matrix cores (v_mfma_i32_32x32x32_i8).
//
// Tiles: 128 x 128 outputs per 256-thread workgroup, K in steps of 64; each of
// the 4 wavefronts owns a 64 x 64 quadrant = 2 x 2 MFMA 32x32 tiles.
//  * A (q) tile 128 x 64 int8 is staged in LDS with each 16-byte chunk
//    byte-transposed into the order the weight expansion produces;
//  * B tile stays packed in LDS (128 rows x 16 bytes); each wavefront expands
//    the 2-bit codes of its fragments to int8 ternary values in registers
//    (shift + mask, then v_perm_b32 as the table {-1, 0, +1, +2}) right before the
//    MFMA, so LDS holds and moves 4x fewer bytes for B;
//  * both operands assign the same k to the same (lane, byte) position, which is
//    all the MFMA needs: the sum over k is order-free in integers;
//  * epilogue: y = fp32(acc * c_m), c_m = (s_x[m] * s_w) / 127 in float64.
// Pages: chenxutan.com sec. 2.3 and sec. 3.1 (BitLinear.forward).
#include "device_common.h"
#include "internal.h"

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int A_STRIDE = 20;  // dwords per A row in LDS (64 bytes + 16 pad)
constexpr int B_STRIDE = 5;   // dwords per B row in LDS (16 bytes + 4 pad)

__global__ __launch_bounds__(256) void gemm_kernel(const int8_t *__restrict__ q,
                                                   const float *__restrict__ s_x,
                                                   const uint8_t *__restrict__ packed,
                                                   const float *__restrict__ s_w, int M, int N, int K,
                                                   float *__restrict__ y, int32_t *__restrict__ acc_out,
                                                   int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint32_t As[BM * A_STRIDE];
    __shared__ uint32_t Bs[BN * B_STRIDE];

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; give each
    // XCD a contiguous range of tiles, walked column-major in groups of 8 M-tiles
    // so that neighbouring workgroups share A rows and B columns in that XCD's L2.
    const int nt = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int q8 = nt / 8, r8 = nt % 8, x = bid % 8;
    const int t = x * q8 + min(x, r8) + bid / 8;  // XCD x owns tiles [x*q8 + min(x,r8), +q8 + (x<r8))
    const int GM = 8;
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsize = min(GM, tiles_m - first_m);
    const int tm = first_m + (t % (GM * tiles_n)) % gsize;
    const int tn = (t % (GM * tiles_n)) / gsize;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int KB = K >> 2;

    v16i acc[2][2];
    #pragma unroll
    for (int i = 0; i < 2; ++i)
        #pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16i{};

    for (int k0 = 0; k0 < K; k0 += BK) {
        // stage A: 128 rows x 4 chunks of 16 bytes, two chunks per thread
        #pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int c = tid + 256 * r;
            const int row = c >> 2, ch = c & 3;
            const int gm = tm * BM + row;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (gm < M) v = *reinterpret_cast<const uint4 *>(q + (size_t)gm * K + k0 + 16 * ch);
            uint4 p;
            transpose4x4(v.x, v.y, v.z, v.w, p.x, p.y, p.z, p.w);
            *reinterpret_cast<uint4 *>(&As[row * A_STRIDE + 4 * ch]) = p;
        }
        // stage B: 128 packed rows x 16 bytes
        if (tid < BN) {
            const int gn = tn * BN + tid;
            uint4 v = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
            if (gn < N) v = *reinterpret_cast<const uint4 *>(packed + (size_t)gn * KB + (k0 >> 2));
            Bs[tid * B_STRIDE + 0] = v.x;
            Bs[tid * B_STRIDE + 1] = v.y;
            Bs[tid * B_STRIDE + 2] = v.z;
            Bs[tid * B_STRIDE + 3] = v.w;
        }
        __syncthreads();
        const int g = lane >> 5, l32 = lane & 31;
        #pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i b[2];
            #pragma unroll
            for (int jn = 0; jn < 2; ++jn) {
                const uint32_t w = Bs[(wn * 64 + jn * 32 + l32) * B_STRIDE + 2 * s + g];
                b[jn] = v4i{(int)codes_to_ternary(codes_i(w, 0)), (int)codes_to_ternary(codes_i(w, 1)),
                            (int)codes_to_ternary(codes_i(w, 2)), (int)codes_to_ternary(codes_i(w, 3))};
            }
            #pragma unroll
            for (int im = 0; im < 2; ++im) {
                const v4i a = *reinterpret_cast<const v4i *>(
                    &As[(wm * 64 + im * 32 + l32) * A_STRIDE + 8 * s + 4 * g]);
                #pragma unroll
                for (int jn = 0; jn < 2; ++jn)
                    acc[im][jn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[jn], acc[im][jn], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // 32x32 accumulator layout: lane -> column l32; register r -> row
    // 8 * (r / 4) + 4 * (lane / 32) + r % 4.
    const float sw = *s_w;
    const int l32 = lane & 31, hi = lane >> 5;
    #pragma unroll
    for (int im = 0; im < 2; ++im) {
        #pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int col = tn * BN + wn * 64 + jn * 32 + l32;
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = tm * BM + wm * 64 + im * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (row < M && col < N) {
                    const size_t o = (size_t)row * N + col;
                    const int v = acc[im][jn][r];
                    y[o] = rescale(v, rescale_factor(s_x[row], sw));
                    if (acc_out) acc_out[o] = v;
                }
            }
        }
    }
}

hipError_t launch_gemm(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                       int64_t M, int64_t N, int64_t K, float *y, int32_t *acc, hipStream_t st) {
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    gemm_kernel<<<dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st>>>(
        q, s_x, packed, s_w, (int)M, (int)N, (int)K, y, acc, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace bitnet
