// Batched decode (up to 16 tokens per pass over the weights) on the matrix cores:
// the same contraction and rescale as the GEMV (pages: chenxutan.com sec. 2.3
// rescale and sec. 3.1 BitLinear.forward), with the products done by
// v_mfma_i32_16x16x64_i8 so that the vector-ALU cost per weight no longer grows
// with the number of tokens.
//
// HBM-bound: every packed weight byte is read once.  Layout of the work:
//  * a wavefront owns RG groups of 16 weight rows and one K slice.  Lane (l16, g)
//    reads, per step, chunk c = c0 + g (16 packed bytes = 64 weights) of row l16 of
//    each group and the 64 q bytes of the same chunk for token l16; tokens past M
//    repeat the last token and their outputs are dropped;
//  * shift + mask regroups a chunk's codes into four 16-byte vectors (vector i,
//    byte 4d + b = code of k = 16d + 4b + i); a 4x4 byte transpose of each 16-byte
//    piece of q puts q in the same order.  Vector i of the weights (A operand: 16
//    rows x 64 k over the 4 lane groups) and vector i of q (B operand: 64 k x 16
//    tokens) make one MFMA: 4 per chunk and row group.  Both operands give a k the
//    same (lane group, byte) position, which is all the sum over k needs;
//  * the codes are c = t + 1: sum_k q t = sum_k q c - sum_k q.  The second term
//    is one more MFMA per vector with an all-ones A operand, shared by the row
//    groups (zero for a clamped chunk past the slice end, whose codes are zeroed);
//  * the loads of step s + 1 are in flight while step s is consumed (two register
//    buffers, no branch in the loop body);
//  * K slices of one row set are summed through LDS;
//  * epilogue: y = fp32(acc * c_m), c_m = (s_x[m] * s_w) / 127 in float64.
#include "device_common.h"
#include "internal.h"

// Weight loads are plain (cached) loads here: one instruction covers half of each
// row's 128-byte line and the next step reads the other half, which a
// nontemporal load would not keep in L2.
#ifndef BITNET_SKINNY_NT
#define BITNET_SKINNY_NT 0
#endif
#ifndef BITNET_SKINNY_WAVES
#define BITNET_SKINNY_WAVES 4096
#endif

namespace bitnet {

typedef int v4i_sk __attribute__((ext_vector_type(4)));

constexpr int kSkinnyNW = 8;          // wavefronts per workgroup (single launches)
#ifndef BITNET_GROUPED_SK_RG
#define BITNET_GROUPED_SK_RG 2
#endif
#ifndef BITNET_GROUPED_SK_NW
#define BITNET_GROUPED_SK_NW 8
#endif
constexpr int kGroupedSkRG = BITNET_GROUPED_SK_RG;   // grouped launches: row groups of 16 per wavefront
constexpr int kGroupedSkNW = BITNET_GROUPED_SK_NW;   // wavefronts per workgroup
#ifndef BITNET_GROUPED_SK_UN
#define BITNET_GROUPED_SK_UN 2
#endif
#ifndef BITNET_GROUPED_SK_NT
#define BITNET_GROUPED_SK_NT 0
#endif
constexpr int kGroupedSkUN = BITNET_GROUPED_SK_UN;   // chunks per lane and step

template <int RG, bool NT>
__device__ __forceinline__ void skinny_tile(const int8_t *__restrict__ q, const float *__restrict__ s_x,
                                            const uint8_t *__restrict__ packed,
                                            const float *__restrict__ s_w, int M, int N, int K,
                                            const OutSpec &out, int32_t *__restrict__ acc_out,
                                            int row_base, int nwaves, int kslices, int *red) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int C = K >> 6;
    const int KB = K >> 2;

    const int rowset = wave / kslices, slice = wave - rowset * kslices;
    const int row0 = row_base + rowset * 16 * RG;
    const int cb = (int)(((int64_t)C * slice) / kslices);
    const int ce = (int)(((int64_t)C * (slice + 1)) / kslices);

    const int8_t *qrow = q + (size_t)min(l16, M - 1) * K;
    const uint8_t *prow[RG];
    #pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int r = row0 + 16 * rg + l16;
        prow[rg] = packed + (size_t)(r < N ? r : 0) * KB;   // rows past N read row 0, dropped
    }

    v4i_sk acc[RG], accq = v4i_sk{0, 0, 0, 0};
    #pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[rg] = v4i_sk{0, 0, 0, 0};

    // step t: lane group g takes chunk cb + 4 t + g; past the slice end the chunk
    // index is clamped (an in-range load) and its codes and ones are zeroed
    const int T = (ce - cb + 3) >> 2;
    const int clast = max(ce - 1, cb);
    uint4 wA[RG], wB[RG], qA[4], qB[4];
    auto issue = [&](uint4 (&w)[RG], uint4 (&qq)[4], int t) {
        const int cc = min(cb + 4 * t + g, clast);
        #pragma unroll
        for (int rg = 0; rg < RG; ++rg) w[rg] = load_weights<NT>(prow[rg] + 16 * cc);
        #pragma unroll
        for (int d = 0; d < 4; ++d) qq[d] = gload16(qrow + 64 * cc + 16 * d);
    };
    auto consume = [&](const uint4 (&w)[RG], const uint4 (&qq)[4], int t) {
        const bool valid = cb + 4 * t + g < ce;
        uint32_t P[4][4];   // P[i][d]: byte b = q of k = 16 d + 4 b + i
        #pragma unroll
        for (int d = 0; d < 4; ++d)
            transpose4x4(qq[d].x, qq[d].y, qq[d].z, qq[d].w, P[0][d], P[1][d], P[2][d], P[3][d]);
        const int one = valid ? 0x01010101 : 0;
        const v4i_sk ones = v4i_sk{one, one, one, one};
        uint32_t wm[RG][4];
        #pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            wm[rg][0] = valid ? w[rg].x : 0u;
            wm[rg][1] = valid ? w[rg].y : 0u;
            wm[rg][2] = valid ? w[rg].z : 0u;
            wm[rg][3] = valid ? w[rg].w : 0u;
        }
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4i_sk b = v4i_sk{(int)P[i][0], (int)P[i][1], (int)P[i][2], (int)P[i][3]};
            accq = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, b, accq, 0, 0, 0);
            #pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const v4i_sk a = v4i_sk{(int)codes_i(wm[rg][0], i), (int)codes_i(wm[rg][1], i),
                                        (int)codes_i(wm[rg][2], i), (int)codes_i(wm[rg][3], i)};
                acc[rg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[rg], 0, 0, 0);
            }
        }
    };
    if (T > 0) {
        issue(wA, qA, 0);
        const int T2 = (T + 1) & ~1;
        for (int t = 0; t < T2 - 2; t += 2) {
            issue(wB, qB, t + 1);
            consume(wA, qA, t);
            issue(wA, qA, t + 2);
            consume(wB, qB, t + 1);
        }
        if (T2 == T) {
            issue(wB, qB, T - 1);
            consume(wA, qA, T - 2);
            consume(wB, qB, T - 1);
        } else {
            consume(wA, qA, T - 1);
        }
    }

    // 16 x 16 accumulator layout: lane -> token l16; register r -> row 4 g + r of the
    // group.  Every row of accq holds sum_k q of the lane's token.
    const float sw = *s_w;
    if (kslices == 1) {
        if (l16 < M) {
            const double cm = rescale_factor(s_x[l16], sw);
            #pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + 16 * rg + 4 * g + r;
                    if (row < N) {
                        const size_t o = (size_t)l16 * N + row;
                        const int v = acc[rg][r] - accq[r];
                        put_y(out, o, row, v, col_factor(out, s_w, row, s_x[l16], cm));
                        if (acc_out) acc_out[o] = v;
                    }
                }
            }
        }
        return;
    }
    #pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        #pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * RG + rg) * 4 + r) * 64 + lane] = acc[rg][r] - accq[r];
    }
    __syncthreads();
    const int rowsets = nwaves / kslices;
    for (int idx = tid; idx < rowsets * RG * 256; idx += nwaves * 64) {
        const int rsi = idx / (RG * 256), rem = idx - rsi * RG * 256;
        const int rg = rem >> 8, r = (rem >> 6) & 3, ln = rem & 63;
        const int tok = ln & 15;
        const int row = row_base + rsi * 16 * RG + 16 * rg + 4 * (ln >> 4) + r;
        if (tok >= M || row >= N) continue;
        int s = 0;
        for (int w = 0; w < kslices; ++w) s += red[(((rsi * kslices + w) * RG + rg) * 4 + r) * 64 + ln];
        const size_t o = (size_t)tok * N + row;
        put_y(out, o, row, s, col_factor(out, s_w, row, s_x[tok], rescale_factor(s_x[tok], sw)));
        if (acc_out) acc_out[o] = s;
    }
}

template <int RG, int NW>
__global__ __launch_bounds__(64 * NW) void skinny_kernel(const int8_t *__restrict__ q,
                                                         const float *__restrict__ s_x,
                                                         const uint8_t *__restrict__ packed,
                                                         const float *__restrict__ s_w, int M, int N, int K,
                                                         const OutSpec out, int32_t *__restrict__ acc_out,
                                                         int kslices) {
    __shared__ int red[NW * RG * 256];
    const int rows_per_block = (NW / kslices) * 16 * RG;
    const int m0 = blockIdx.y * 16;   // tiles of 16 tokens (one for M <= 16)
    skinny_tile<RG, BITNET_SKINNY_NT != 0>(q + (size_t)m0 * K, s_x + m0, packed, s_w, min(16, M - m0), N, K,
                                           out_offset(out, (size_t)m0 * N), acc_out ? acc_out + (size_t)m0 * N : nullptr,
                                           blockIdx.x * rows_per_block, NW, kslices, red);
}

template <int RG>
static void launch_rg(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w, int64_t M,
                      int64_t N, int64_t K, const OutSpec &y, int32_t *acc, int ks, hipStream_t st) {
    constexpr int NW = kSkinnyNW;
    const int rows_per_block = (NW / ks) * 16 * RG;
    const unsigned blocks = (unsigned)((N + rows_per_block - 1) / rows_per_block);
    const unsigned mtiles = (unsigned)((M + 15) / 16);
    skinny_kernel<RG, NW><<<dim3(blocks, mtiles), dim3(64 * NW), 0, st>>>(q, s_x, packed, s_w, (int)M, (int)N,
                                                                          (int)K, y, acc, ks);
}

// Estimated time (us) of launch_skinny: the first 16 tokens stream the weights at
// about 3.5 TB/s plus 5 us; each further 16-token tile (a concurrent re-read of the
// weights) adds about W / 4 TB/s + 1.8 us (measured on M = 16 .. 256 against six
// shapes from 2560 x 2560 to 8192 x 28672).
double skinny_estimate_us(int64_t M, int64_t N, int64_t K) {
    const double w = (double)N * (double)K / 4.0;   // packed bytes
    const int64_t tiles = (M + 15) / 16;
    return w / 3.5e6 + 5.0 + (double)(tiles - 1) * (w / 4.0e6 + 1.8);
}

hipError_t launch_skinny(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                         int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    // Rows per wavefront (16 RG) against parallelism: the largest RG whose launch,
    // with K split over up to 8 wavefronts of a workgroup (at least 8 chunks per
    // slice), still reaches 2048 wavefronts (one workgroup per CU); more row groups
    // per wavefront share each q load.
    const int C = (int)(K / 64);
    int rg = 1, ks = 1;
    for (int r = 4; r >= 1; r >>= 1) {
        const int64_t groups = (N + 16 * r - 1) / (16 * r);
        int k = 1;
        while (k < kSkinnyNW && groups * k < BITNET_SKINNY_WAVES && C / (2 * k) >= 8) k *= 2;
        rg = r;
        ks = k;
        if (groups * k >= 2048) break;
    }
    if (rg == 4) launch_rg<4>(q, s_x, packed, s_w, M, N, K, y, acc, ks, st);
    else if (rg == 2) launch_rg<2>(q, s_x, packed, s_w, M, N, K, y, acc, ks, st);
    else launch_rg<1>(q, s_x, packed, s_w, M, N, K, y, acc, ks, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LDS-staged variant (grouped launches): the NW wavefronts of a workgroup walk the
// whole K of NW x 16 RG rows (8 x 32 = 256: measured against 4 x 32, 16 x 32 and
// 8 x 64, it stages each q for the most rows without starving the grid).  The q of a
// K segment (all tokens) is loaded once per
// workgroup, byte-transposed once and kept in LDS in MFMA B-operand order (chunk,
// vector i, token: 16 bytes each), so the main loop issues only weight loads and
// reads its B operands from LDS; sum_k q is formed while staging.  A segment is as
// long as the LDS budget allows for the problem's M tokens: the whole K for every
// decode-step shape up to 12 tokens; one barrier pair per segment.
constexpr int kSkLdsBudget = 64 * 1024;

// A staged chunk takes 64 M bytes of q plus 16 bytes of padding: the threads that
// stage consecutive chunks (and the lane groups that read them) then fall 4 banks
// apart instead of on the same banks.
__host__ __device__ __forceinline__ int sk_chunk_dw(int M) { return 16 * M + 4; }

// Segment length in 64-weight chunks for M tokens: all of K if its staged q fits the
// budget, else the fewest equal segments, each a multiple of 8 chunks (one step).
__host__ __device__ __forceinline__ int sk_segment_chunks(int C, int M) {
    const int max_seg = (kSkLdsBudget / (4 * sk_chunk_dw(M))) & ~7;
    if (C <= max_seg) return C;
    const int nseg = (C + max_seg - 1) / max_seg;
    return (((C + nseg - 1) / nseg) + 7) & ~7;
}

template <int RG, int UN, bool NT>
__device__ __forceinline__ void skinny_lds_tile(const int8_t *__restrict__ q, const float *__restrict__ s_x,
                                                const uint8_t *__restrict__ packed,
                                                const float *__restrict__ s_w, int M, int N, int K,
                                                const OutSpec &out, int32_t *__restrict__ acc_out,
                                                int row_base, uint32_t *qs, int *sq) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int C = K >> 6;
    const int KB = K >> 2;
    const int row0 = row_base + wave * 16 * RG;
    const int tok = min(l16, M - 1);
    const int seg_chunks = sk_segment_chunks(C, M);

    const uint8_t *prow[RG];
    #pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int r = row0 + 16 * rg + l16;
        prow[rg] = packed + (size_t)(r < N ? r : 0) * KB;   // rows past N read row 0, dropped
    }

    v4i_sk acc[RG];
    #pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[rg] = v4i_sk{0, 0, 0, 0};
    if (tid < 16) sq[tid] = 0;

    for (int s0 = 0; s0 < C; s0 += seg_chunks) {
        const int sc = min(seg_chunks, C - s0);
        // step t: lane group g takes local chunks 4 UN t + 4 u + g, u < UN (the UN loads
        // of a row group are back to back: 64 UN contiguous bytes of each row); chunks
        // past the segment are clamped to an in-range load and zeroed
        const int T = (sc + 4 * UN - 1) / (4 * UN);
        uint4 wA[UN][RG], wB[UN][RG];
        auto issue = [&](uint4 (&w)[UN][RG], int t) {
            #pragma unroll
            for (int u = 0; u < UN; ++u) {
                const int cc = s0 + min(4 * UN * t + 4 * u + g, sc - 1);
                #pragma unroll
                for (int rg = 0; rg < RG; ++rg) w[u][rg] = load_weights<NT>(prow[rg] + 16 * cc);
            }
        };
        auto consume = [&](const uint4 (&w)[UN][RG], int t) {
            #pragma unroll
            for (int u = 0; u < UN; ++u) {
                const int cl = 4 * UN * t + 4 * u + g;
                const bool valid = cl < sc;
                const uint32_t *src = qs + min(cl, sc - 1) * sk_chunk_dw(M) + tok * 4;
                uint32_t wm[RG][4];
                #pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                    wm[rg][0] = valid ? w[u][rg].x : 0u;
                    wm[rg][1] = valid ? w[u][rg].y : 0u;
                    wm[rg][2] = valid ? w[u][rg].z : 0u;
                    wm[rg][3] = valid ? w[u][rg].w : 0u;
                }
                #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4i_sk b = *reinterpret_cast<const v4i_sk *>(src + i * M * 4);
                    #pragma unroll
                    for (int rg = 0; rg < RG; ++rg) {
                        const v4i_sk a = v4i_sk{(int)codes_i(wm[rg][0], i), (int)codes_i(wm[rg][1], i),
                                                (int)codes_i(wm[rg][2], i), (int)codes_i(wm[rg][3], i)};
                        acc[rg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[rg], 0, 0, 0);
                    }
                }
            }
        };
        // the segment's first weight loads go out before the staging of q
        if (T > 0) issue(wA, 0);

        // ---- stage the segment's q: (token m, chunk c) per thread, 64 contiguous bytes
        __syncthreads();   // previous segment's LDS reads done; sq initialised
        for (int idx = tid; idx < M * sc; idx += blockDim.x) {
            const int m = idx / sc, c = idx - m * sc;
            const int8_t *src = q + (size_t)m * K + 64 * (s0 + c);
            uint4 v[4];
            #pragma unroll
            for (int d = 0; d < 4; ++d) v[d] = gload16(src + 16 * d);
            uint32_t P[4][4];   // P[i][d]: byte b = q of k = 16 d + 4 b + i
            int sm = 0;
            #pragma unroll
            for (int d = 0; d < 4; ++d) {
                transpose4x4(v[d].x, v[d].y, v[d].z, v[d].w, P[0][d], P[1][d], P[2][d], P[3][d]);
                sm = dot4(v[d].x, 0x01010101u, sm);
                sm = dot4(v[d].y, 0x01010101u, sm);
                sm = dot4(v[d].z, 0x01010101u, sm);
                sm = dot4(v[d].w, 0x01010101u, sm);
            }
            #pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4 *>(qs + c * sk_chunk_dw(M) + (i * M + m) * 4) =
                    make_uint4(P[i][0], P[i][1], P[i][2], P[i][3]);
            if (sm != 0) atomicAdd(&sq[m], sm);
        }
        __syncthreads();

        // pairs of steps, no branch in the loop body; the last one or two peeled
        if (T > 0) {
            const int T2 = (T + 1) & ~1;
            for (int t = 0; t < T2 - 2; t += 2) {
                issue(wB, t + 1);
                consume(wA, t);
                issue(wA, t + 2);
                consume(wB, t + 1);
            }
            if (T2 == T) {
                issue(wB, T - 1);
                consume(wA, T - 2);
                consume(wB, T - 1);
            } else {
                consume(wA, T - 1);
            }
        }
    }

    // 16 x 16 accumulator layout: lane -> token l16; register r -> row 4 g + r
    if (l16 < M) {
        const float sw = *s_w;
        const double cm = rescale_factor(s_x[l16], sw);
        const int sqm = sq[l16];
        #pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + 16 * rg + 4 * g + r;
                if (row < N) {
                    const size_t o = (size_t)l16 * N + row;
                    const int v = acc[rg][r] - sqm;
                    put_y(out, o, row, v, col_factor(out, s_w, row, s_x[l16], cm));
                    if (acc_out) acc_out[o] = v;
                }
            }
        }
    }
}

// Grouped decode on the matrix cores: block -> (descriptor, row block of NW x 16 RG
// rows) through the plan's block table; every descriptor has M <= 16.
__global__ __launch_bounds__(64 * kGroupedSkNW) void skinny_grouped_kernel(const uint8_t *__restrict__ plan) {
    extern __shared__ __attribute__((aligned(16))) uint32_t qs[];   // staged q of one segment
    __shared__ int sq[16];
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[blockIdx.x];
    const LinearDescDev d = reinterpret_cast<const LinearDescDev *>(plan + h->desc_offset)[e.desc];
    skinny_lds_tile<kGroupedSkRG, kGroupedSkUN, BITNET_GROUPED_SK_NT != 0>(d.q, d.s_x, d.packed, d.s_w, d.M, d.N, d.K, OutSpec{d.y, nullptr, 0, d.w_group}, d.acc,
                                                         (int)e.local * kGroupedSkNW * 16 * kGroupedSkRG, qs, sq);
}

uint32_t skinny_grouped_rows_per_block() { return kGroupedSkNW * 16 * kGroupedSkRG; }
uint32_t skinny_grouped_lds_bytes(int64_t M, int64_t K) {
    return (uint32_t)(sk_segment_chunks((int)(K / 64), (int)M) * sk_chunk_dw((int)M) * 4);
}

hipError_t launch_skinny_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, hipStream_t st) {
    skinny_grouped_kernel<<<dim3(blocks), dim3(64 * kGroupedSkNW), lds_bytes, st>>>(reinterpret_cast<const uint8_t *>(plan_dev));
    return hipGetLastError();
}

}  // namespace bitnet
