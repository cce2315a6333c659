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

static bool skinny2_single_ok(const int8_t *q, const uint8_t *packed, int64_t M, int64_t N, int64_t K, const OutSpec &y);
static hipError_t launch_skinny2_single(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                                        int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st);

hipError_t launch_skinny(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                         int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    // Many rows (at least two 256-row workgroups per CU): the line-granular kernel of the
    // grouped launches, one 256-row block per workgroup, all tokens at once.
    if (skinny2_single_ok(q, packed, M, N, K, y)) return launch_skinny2_single(q, s_x, packed, s_w, M, N, K, y, acc, st);
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
#ifndef BITNET_SK_LDS_KB
#define BITNET_SK_LDS_KB 64
#endif
constexpr int kSkLdsBudget = BITNET_SK_LDS_KB * 1024;

// A staged chunk takes 64 M bytes of q plus 16 bytes of padding: the threads that
// stage consecutive chunks (and the lane groups that read them) then fall 4 banks
// apart instead of on the same banks.
__host__ __device__ __forceinline__ int sk_chunk_dw(int M) { return 16 * M + 4; }

// Segment length in 64-weight chunks for M tokens: all of K if its staged q fits the
// budget, else the fewest equal segments, each a multiple of 8 chunks (one step).
// grp: the group-wise path of the line-granular kernel, which keeps less staged q
// (kSkLdsBudgetGrp) so that two of its workgroups fit a CU beside their larger static LDS.
constexpr int kSkLdsBudgetGrp = 48 * 1024;
__host__ __device__ __forceinline__ int sk_segment_chunks(int C, int M, bool grp = false) {
    const int max_seg = ((grp ? kSkLdsBudgetGrp : kSkLdsBudget) / (4 * sk_chunk_dw(M))) & ~7;
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

// ---------------------------------------------------------------------------
// Line-granular grouped variant (the one grouped launches use).  The weights are
// read in whole 128-byte lines: the 8 lanes of an octet take the 8 16-byte pieces of
// one line of one row, so one load instruction covers 8 rows x 128 bytes, and the
// loads are nontemporal.  A wavefront then regroups each step (one line of each of
// its rows) into MFMA operands through a small LDS buffer of its own: lane
// (row i, piece p) writes its 16 bytes, lane (row r16, lane group g) reads pieces 2g
// and 2g + 1 of row r16 back (one LDS write and one read per 16 bytes, no barrier:
// a wavefront's LDS accesses are carried out in order).
//  * MFMA f (0..7) of a step takes, in lane (r16, g), dword f of those 32 bytes:
//    16 codes of row r16 at k = 16 D + 4b + i (D = the dword's 16-weight block, byte
//    b), spread by shift + mask into four dwords (dword i, byte b = code of
//    k = 16 D + 4b + i) as the A operand.  The B operand, lane (token, g), holds the
//    16 q values of the same block in the same order (a 4x4 byte transpose made once
//    while staging q), so the k of every (lane group, byte) position agrees.
//  * Rows whose packed rows start mid-line (K = 6912: every other row starts 64 bytes
//    into a line) are loaded line-aligned, and a step's window of 8 pieces is shifted
//    by the rows' offset.  The rows of one 16-row block share their offset: block beta
//    holds rows 16 P (beta / P) + beta % P + P i, P = the period of the offsets (1, 2,
//    4 or 8 rows), and a wavefront takes blocks w and w + 8 (one offset).  Pieces
//    outside the row (or the staged K segment) are written as zero codes.
//  * The codes are c = t + 1: sum q t = sum q c - sum q, sum q formed while staging.
//  * The results of the workgroup's 256 rows go through LDS and are stored as whole
//    row segments per token.
constexpr int kSk2NW = 8;       // wavefronts per workgroup
constexpr int kSk2RB = 2;       // 16-row blocks per wavefront
constexpr int kSk2TDw = 36;     // dwords per row of a wavefront's regrouping buffer (32 + 4 pad)
constexpr int kSk2Rows = kSk2NW * kSk2RB * 16;
constexpr int kSk2YStride = kSk2Rows + 1;   // ints per token row of the staged results
constexpr int kSk2Items = (kSkLdsBudget / 64 + 64 * kSk2NW - 1) / (64 * kSk2NW);   // staged items per thread
#ifndef SK2_PRE
#define SK2_PRE 1       // steps of weight loads issued before the q staging (1 or 2)
#endif
#ifndef SK2_WAVES
#define SK2_WAVES 4     // wavefronts per SIMD the register allocation aims at
#endif

// GRP: group-wise weight scales (d.w_group = G below K, a multiple of 64; s_w is
// [N][K / G]).  Then MFMA f of a step takes piece f (one 64-weight chunk, a single
// group's) in every lane group: lane (row r16, group g) holds dword g of piece f, and
// the B operand block g of that chunk.  After the MFMA of a group's last chunk its
// products, less the group's sum of q (per-chunk sums kept while staging), are scaled
// by the rows' group scales into float64 accumulators; the scales travel with the
// weights (loaded beside each piece, regrouped through LDS with them).
// IT (with GRP): also keep each row's exact integer sum of the group-wise problems,
// for their int32 acc output; without it only the problems with one group (whose
// float64 sum is that integer exactly) have acc.
template <bool NT, bool GRP, bool IT = true>
__device__ __forceinline__ void skinny2_tile(const LinearDescDev &d, int row_base, uint32_t *qs, uint32_t *tb,
                                             float *tsc, int *sq, double *cms) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4, o = lane >> 3, l8 = lane & 7;
    const int M = d.M, N = d.N, K = d.K;
    const int C = K >> 6, KB = K >> 2;
    // rows whose packed rows start at the same position within a 128-byte line recur
    // every P rows (KB is a multiple of 16)
    const int kbm = KB & 127;
    const int P = kbm == 0 ? 1 : 128 / (kbm & -kbm);
    int rb0[kSk2RB];
    #pragma unroll
    for (int b = 0; b < kSk2RB; ++b) {
        const int beta = wave + kSk2NW * b;
        rb0[b] = row_base + 16 * P * (beta / P) + beta % P;
    }
    // pieces (16 bytes) between the start of the line and the rows' first byte
    const int off = (int)(((uintptr_t)(d.packed + (size_t)rb0[0] * KB) & 127) >> 4);
    const uint8_t *prow[kSk2RB][2];
    // GRP: chunks per scale group, groups per row.  A problem without group-wise scales
    // (dg false: one scale per tensor or per output channel) runs the same path with one
    // group of all of K and its own rescale at the end.
    const bool dg = GRP && d.w_group > 0 && d.w_group < K;
    const int gc = dg ? d.w_group >> 6 : C, ng = dg ? K / d.w_group : 1;
    #pragma unroll
    for (int b = 0; b < kSk2RB; ++b)
        #pragma unroll
        for (int h = 0; h < 2; ++h)
            prow[b][h] = d.packed + (size_t)min(rb0[b] + P * (8 * h + o), N - 1) * KB;   // rows past N: dropped

    v4i_sk acc[kSk2RB];
    #pragma unroll
    for (int b = 0; b < kSk2RB; ++b) acc[b] = v4i_sk{0, 0, 0, 0};
    // GRP: sum over the groups done of (products - sum q) s_g and of (products - sum q)
    double facc[GRP ? kSk2RB : 1][4];
    int itot[GRP && IT ? kSk2RB : 1][4];
    int sqrun = 0;   // GRP: sum of q over the current group's chunks so far (lane's token)
    if (GRP) {
        #pragma unroll
        for (int b = 0; b < kSk2RB; ++b)
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                facc[b][r] = 0.0;
                if (IT) itot[b][r] = 0;
            }
    }
    if (tid < 16) sq[tid] = 0;
    const int tokc = min(l16, M - 1);   // tokens past M repeat the last one (outputs dropped)
    // plain kernel: the epilogue's scales (the lane's token's s_x; the per-tensor s_w
    // through the scalar path), read before the weight stream so that their latency is
    // not paid after the last step (1.9 us per 8-token decode step).  The group-wise
    // kernel reads them at the end: holding them costs it spills.
    const float sx_early = GRP ? 0.0f : d.s_x[tokc];
    const float sw_early = GRP ? 0.0f : *(const __attribute__((address_space(4))) float *)d.s_w;
    uint32_t *tw = tb + wave * 16 * kSk2TDw;
    float *ts = GRP ? tsc + wave * kSk2RB * 8 * 16 : nullptr;   // GRP: [block][piece][row] scales of a step
    static_assert(kSk2Items * kSk2NW * 64 * 64 >= kSkLdsBudget, "one staging pass covers a segment");
    const int seg_chunks = sk_segment_chunks(C, M, GRP);
    const int cdw = sk_chunk_dw(M);
    int *sqc = reinterpret_cast<int *>(qs + seg_chunks * cdw);   // GRP: [token][chunk] sums of q

    for (int s0 = 0; s0 < C; s0 += seg_chunks) {
        const int sc = min(seg_chunks, C - s0), s1 = s0 + sc;
        // step t: piece l8 of line t (from the rows' line start) is chunk 8t + l8 - off;
        // the steps whose window [8t - off, 8t + 8 - off) meets [s0, s1)
        const int t0 = (s0 + off) >> 3, T = ((s1 + off + 7) >> 3) - t0;
        struct WBuf { uint4 w[kSk2RB][2]; float s[GRP ? kSk2RB : 1][2]; };
        WBuf wA, wB;
        auto issue = [&](WBuf &w, int t) {
            const int c = min(max(8 * (t0 + t) + l8 - off, s0), s1 - 1);
            const int grp = GRP ? c / gc : 0;
            #pragma unroll
            for (int b = 0; b < kSk2RB; ++b)
                #pragma unroll
                for (int h = 0; h < 2; ++h) {
                    w.w[b][h] = load_weights<NT>(prow[b][h] + 16 * c);
                    // GRP: the loading lane's row's scale of the chunk's group
                    if (GRP) w.s[b][h] = dg ? d.s_w[(size_t)min(rb0[b] + P * (8 * h + o), N - 1) * ng + grp] : 1.0f;
                }
        };
        auto consume = [&](const WBuf &w, int t) {
            const int cw = 8 * (t0 + t) - off;        // first chunk of the window
            const bool valid = cw + l8 >= s0 && cw + l8 < s1;
            // regroup both blocks through the wavefront's buffer (block 1 written after
            // block 0 is read back).  Plain: pw[b][f] = dword f of pieces 2g, 2g + 1 of
            // row l16; GRP: dword g of piece f (pieces stored dword-major)
            uint32_t pw[kSk2RB][8];
            #pragma unroll
            for (int b = 0; b < kSk2RB; ++b) {
                #pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 v = valid ? w.w[b][h] : make_uint4(0u, 0u, 0u, 0u);
                    if (GRP) {
                        uint32_t *dst = tw + (8 * h + o) * kSk2TDw + l8;
                        dst[0] = v.x; dst[8] = v.y; dst[16] = v.z; dst[24] = v.w;
                        ts[(b * 8 + l8) * 16 + 8 * h + o] = w.s[b][h];
                    } else {
                        *reinterpret_cast<uint4 *>(tw + (8 * h + o) * kSk2TDw + 4 * l8) = v;
                    }
                }
                const uint4 a0 = *reinterpret_cast<const uint4 *>(tw + l16 * kSk2TDw + 8 * g);
                const uint4 a1 = *reinterpret_cast<const uint4 *>(tw + l16 * kSk2TDw + 8 * g + 4);
                pw[b][0] = a0.x; pw[b][1] = a0.y; pw[b][2] = a0.z; pw[b][3] = a0.w;
                pw[b][4] = a1.x; pw[b][5] = a1.y; pw[b][6] = a1.z; pw[b][7] = a1.w;
            }
            #pragma unroll
            for (int f = 0; f < 8; ++f) {
                // B operand.  Plain: chunk cw + 2g + f / 4, block f % 4; GRP: chunk cw + f,
                // block g (clamped into the segment where the codes are zero)
                const int craw = GRP ? cw + f : cw + 2 * g + (f >> 2);
                const int cl = min(max(craw - s0, 0), sc - 1);
                const v4i_sk bq = *reinterpret_cast<const v4i_sk *>(qs + cl * cdw + ((GRP ? g : (f & 3)) * M + tokc) * 4);
                #pragma unroll
                for (int b = 0; b < kSk2RB; ++b) {
                    const uint32_t x = pw[b][f];
                    const v4i_sk a = v4i_sk{(int)codes_i(x, 0), (int)codes_i(x, 1), (int)codes_i(x, 2), (int)codes_i(x, 3)};
                    acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bq, acc[b], 0, 0, 0);
                }
                if (GRP && craw >= s0 && craw < s1) {
                    sqrun += sqc[tokc * seg_chunks + cl];
                    if ((craw + 1) % gc == 0) {
                        // the group's last chunk: fold its products into the accumulators
                        #pragma unroll
                        for (int b = 0; b < kSk2RB; ++b) {
                            const float4 s4 = *reinterpret_cast<const float4 *>(ts + (b * 8 + f) * 16 + 4 * g);
                            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
                            #pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int pr = acc[b][r] - sqrun;   // |pr| <= 127 G
                                facc[b][r] += (double)pr * (double)sv[r];
                                if (IT) itot[b][r] += pr;
                            }
                            acc[b] = v4i_sk{0, 0, 0, 0};
                        }
                        sqrun = 0;
                    }
                }
            }
        };
        // ---- stage the segment's q: (token m, chunk c) items, several per thread and
        // pass; block D of a chunk (16 values) transposed as the B operand of the blocks'
        // MFMAs (GRP: and each item's sum of q kept per chunk).  The first pass's q loads
        // go out before the segment's first weight loads, so that the staging waits for
        // its own (L2-resident) data only, not for the weights.
        auto stage_item = [&](int idx, const uint4 (&v)[4]) {
            const int m = idx / sc, c = idx - m * sc;
            int sm = 0;
            #pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t p0, p1, p2, p3;
                transpose4x4(v[j].x, v[j].y, v[j].z, v[j].w, p0, p1, p2, p3);
                *reinterpret_cast<uint4 *>(qs + c * cdw + (j * M + m) * 4) = make_uint4(p0, p1, p2, p3);
                sm = dot4(v[j].x, 0x01010101u, sm);
                sm = dot4(v[j].y, 0x01010101u, sm);
                sm = dot4(v[j].z, 0x01010101u, sm);
                sm = dot4(v[j].w, 0x01010101u, sm);
            }
            if (GRP) sqc[m * seg_chunks + c] = sm;
            if (sm != 0) atomicAdd(&sq[m], sm);
        };
        const int items = M * sc, nth = (int)blockDim.x;
        // item idx (clamped: a duplicate is loaded, not staged) into v
        auto load_item = [&](int idx, uint4 (&v)[4]) {
            const int i = min(idx, items - 1);
            const int m = i / sc, c = i - m * sc;
            const int8_t *src = d.q + (size_t)m * K + 64 * (s0 + c);
            #pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = gload16(src + 16 * j);
        };
        // A segment holds fewer than kSk2Items nth items (the LDS budget over 16 M + 4
        // dwords per chunk is under budget / 64 / M chunks), so one pass stages it.  The
        // barriers wait for the LDS accesses only (an s_barrier after lgkmcnt(0)):
        // __syncthreads() would also wait for the weight loads in flight.
        uint4 v[kSk2Items][4];
        #pragma unroll
        for (int u = 0; u < kSk2Items; ++u) load_item(tid + u * nth, v[u]);
        issue(wA, 0);
        if (SK2_PRE > 1) issue(wB, 1);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // previous segment's LDS reads done
        #pragma unroll
        for (int u = 0; u < kSk2Items; ++u)
            if (tid + u * nth < items) stage_item(tid + u * nth, v[u]);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

        // pairs of steps, no branch in the loop body; the last one to three peeled
        if (SK2_PRE > 1) {
            // steps t and t + 1 are in flight at the top of every iteration
            int t = 0;
            for (; t + 3 < T; t += 2) {
                consume(wA, t);
                issue(wA, t + 2);
                consume(wB, t + 1);
                issue(wB, t + 3);
            }
            if (T - t == 3) {
                consume(wA, t);
                issue(wA, t + 2);
                consume(wB, t + 1);
                consume(wA, t + 2);
            } else if (T - t == 2) {
                consume(wA, t);
                consume(wB, t + 1);
            } else {
                consume(wA, t);
            }
        } else {
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

    // ---- epilogue.  Plain: acc (16 x 16 layout: lane -> token l16, register r -> row
    // 4g + r of the block) less sum q into LDS as [token][row of the workgroup], then whole
    // row segments per token, rescaled.  GRP: the lane forms y itself, y = fp32((sum_g
    // (acc_g - sum_g q) s_g) s_x / 127 (+ bias)), and stages its bits beside the exact
    // integer sums.
    __syncthreads();   // every wavefront done with the staged q
    // rows of kSk2YStride ints: the 16 tokens of one row fall on 16 different banks
    int *ys = reinterpret_cast<int *>(qs);
    int *ys2 = ys + 16 * kSk2YStride;   // dg: the integer sums
    if (l16 < M) {
        const int sqm = sq[l16];
        #pragma unroll
        for (int b = 0; b < kSk2RB; ++b)
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = rb0[b] - row_base + P * (4 * g + r);
                if (dg) {
                    const int row = min(row_base + rl, N - 1);
                    double yv = (facc[b][r] * (double)d.s_x[l16]) / 127.0;
                    if (d.bias) yv += (double)d.bias[row];
                    ys[l16 * kSk2YStride + rl] = (int)__float_as_uint((float)yv);
                    ys2[l16 * kSk2YStride + rl] = IT ? itot[b][r] : 0;
                } else {
                    // GRP: one group of all of K with scale 1, its float64 sum exact
                    ys[l16 * kSk2YStride + rl] = GRP ? (IT ? itot[b][r] : (int)facc[b][r]) : acc[b][r] - sqm;
                }
            }
    }
    if (!dg && tid < M) {
        const float sxm = GRP ? d.s_x[tid] : sx_early;   // tid < 16: token tid
        cms[tid] = rescale_factor(sxm, GRP ? *d.s_w : sw_early);
        cms[16 + tid] = (double)sxm;
    }
    __syncthreads();
    const OutSpec out = d.out();
    for (int idx = tid; idx < M * kSk2Rows; idx += blockDim.x) {
        const int m = idx / kSk2Rows, rr = idx - m * kSk2Rows, row = row_base + rr;
        if (row < N) {
            const size_t o2 = (size_t)m * N + row;
            if (dg) {
                const float yf = __uint_as_float((uint32_t)ys[m * kSk2YStride + rr]);
                if (out.bf16) reinterpret_cast<uint16_t *>(out.y)[o2] = bf16_rne(yf);
                else reinterpret_cast<float *>(out.y)[o2] = yf;
                if (d.acc) d.acc[o2] = ys2[m * kSk2YStride + rr];
            } else {
                const int v = ys[m * kSk2YStride + rr];
                put_y(out, o2, row, v, col_factor(out, d.s_w, row, (float)cms[16 + m], cms[m]));
                if (d.acc) d.acc[o2] = v;
            }
        }
    }
}

#ifndef BITNET_SKINNY_V2
#define BITNET_SKINNY_V2 1
#endif

// Grouped decode on the matrix cores: block -> (descriptor, row block of 256 rows)
// through the plan's block table; every descriptor has M <= 16.
__global__ __launch_bounds__(64 * kGroupedSkNW) void skinny_grouped_kernel(const uint8_t *__restrict__ plan) {
    extern __shared__ __attribute__((aligned(16))) uint32_t qs[];   // staged q of one segment
    __shared__ int sq[16];
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[blockIdx.x];
    const LinearDescDev d = reinterpret_cast<const LinearDescDev *>(plan + h->desc_offset)[e.desc];
    skinny_lds_tile<kGroupedSkRG, kGroupedSkUN, BITNET_GROUPED_SK_NT != 0>(d.q, d.s_x, d.packed, d.s_w, d.M, d.N, d.K, d.out(), d.acc,
                                                         (int)e.local * kGroupedSkNW * 16 * kGroupedSkRG, qs, sq);
}

// GRP: the plan has problems with group-wise weight scales, which take the group-wise
// tile; plans without them use the kernel without it.
template <bool GRP, bool IT = true>
__global__ __launch_bounds__(64 * kSk2NW) __attribute__((amdgpu_waves_per_eu(SK2_WAVES))) void skinny2_grouped_kernel(const uint8_t *__restrict__ plan) {
    extern __shared__ __attribute__((aligned(16))) uint32_t qs[];   // staged q of one segment; results
    __shared__ __attribute__((aligned(16))) uint32_t tb[kSk2NW * 16 * kSk2TDw];
    __shared__ __attribute__((aligned(16))) float tsc[GRP ? kSk2NW * kSk2RB * 8 * 16 : 4];
    __shared__ int sq[16];
    __shared__ double cms[32];   // per token: c_m, then s_x
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[blockIdx.x];
    const LinearDescDev d = reinterpret_cast<const LinearDescDev *>(plan + h->desc_offset)[e.desc];
    skinny2_tile<true, GRP, IT>(d, (int)e.local * kSk2Rows, qs, tb, tsc, sq, cms);
}

static_assert(kSk2Rows == kGroupedSkNW * 16 * kGroupedSkRG, "both grouped variants take 256-row blocks");

// The same kernel for one matrix (bitnet_linear with 2..16 tokens and many rows):
// workgroup b takes rows 256 b .. 256 b + 255.
__global__ __launch_bounds__(64 * kSk2NW) __attribute__((amdgpu_waves_per_eu(SK2_WAVES))) void skinny2_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s_x, const uint8_t *__restrict__ packed,
    const float *__restrict__ s_w, int M, int N, int K, const OutSpec out, int32_t *__restrict__ acc) {
    extern __shared__ __attribute__((aligned(16))) uint32_t qs[];
    __shared__ __attribute__((aligned(16))) uint32_t tb[kSk2NW * 16 * kSk2TDw];
    __shared__ int sq[16];
    __shared__ double cms[32];   // per token: c_m, then s_x
    const LinearDescDev d{q, s_x, packed, s_w, out.y, acc, M, N, K, out.w_group, out.bias, out.bf16, 0};
    skinny2_tile<true, false>(d, (int)blockIdx.x * kSk2Rows, qs, tb, nullptr, sq, cms);
}

// At least 2 workgroups per CU of a 256-CU part, up to 16 tokens, whole 64-weight
// chunks and 16-byte aligned q / packed rows (the grouped launches' preconditions);
// group-wise weight scales take the GEMV.
constexpr int64_t kSk2SingleMinRows = 512 * (int64_t)kSk2Rows;

static bool skinny2_single_ok(const int8_t *q, const uint8_t *packed, int64_t M, int64_t N, int64_t K, const OutSpec &y) {
    return BITNET_SKINNY_V2 && M >= 1 && M <= 16 && N >= kSk2SingleMinRows && N < ((int64_t)1 << 31) && K % 64 == 0 &&
           K < ((int64_t)1 << 30) && reinterpret_cast<uintptr_t>(q) % 16 == 0 && reinterpret_cast<uintptr_t>(packed) % 16 == 0 &&
           (y.w_group == 0 || y.w_group == K);
}

static hipError_t launch_skinny2_single(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                                        int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    const unsigned blocks = (unsigned)((N + kSk2Rows - 1) / kSk2Rows);
    skinny2_kernel<<<dim3(blocks), dim3(64 * kSk2NW), skinny_grouped_lds_bytes(M, K), st>>>(
        q, s_x, packed, s_w, (int)M, (int)N, (int)K, y, acc);
    return hipGetLastError();
}

uint32_t skinny_grouped_rows_per_block() { return kGroupedSkNW * 16 * kGroupedSkRG; }
uint32_t skinny_grouped_lds_bytes(int64_t M, int64_t K, bool grp) {
    const int seg = sk_segment_chunks((int)(K / 64), (int)M, grp);
    // group-wise problems also keep each (token, chunk) sum of q after the staged chunks
    const uint32_t stage = (uint32_t)(seg * sk_chunk_dw((int)M) * 4 + (grp ? (int)M * seg * 4 : 0));
    // the line-granular variant also keeps the results of its 256 rows there (16 tokens;
    // group-wise: the fp32 y and the integer sums)
    return BITNET_SKINNY_V2 ? std::max<uint32_t>(stage, (grp ? 2u : 1u) * 16u * kSk2YStride * 4u) : stage;
}

hipError_t launch_skinny_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, bool grp, bool grp_acc,
                                 hipStream_t st) {
    const uint8_t *p = reinterpret_cast<const uint8_t *>(plan_dev);
    // group-wise plans: the integer sums only when a group-wise problem asks for acc
    // (8 registers fewer, no spills at 4 waves per SIMD: 8-token decode step with
    // group-128 scales 188.5 -> 178.8 us)
    if (grp && grp_acc) skinny2_grouped_kernel<true, true><<<dim3(blocks), dim3(64 * kSk2NW), lds_bytes, st>>>(p);
    else if (grp) skinny2_grouped_kernel<true, false><<<dim3(blocks), dim3(64 * kSk2NW), lds_bytes, st>>>(p);
    else if (BITNET_SKINNY_V2) skinny2_grouped_kernel<false><<<dim3(blocks), dim3(64 * kSk2NW), lds_bytes, st>>>(p);
    else skinny_grouped_kernel<<<dim3(blocks), dim3(64 * kGroupedSkNW), lds_bytes, st>>>(p);
    return hipGetLastError();
}

}  // namespace bitnet
