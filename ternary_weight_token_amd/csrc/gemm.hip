// Prefill GEMM (M > 16): the same contraction and rescale as the GEMV, as a dense
// int8 x ternary -> int32 product on the matrix cores (v_mfma_i32_16x16x64_i8).
// Pages: chenxutan.com sec. 2.3 (rescale) and sec. 3.1 (BitLinear.forward).
//
// Workgroup = WM x WN wavefronts; a wavefront owns TM x TN MFMA tiles of 16 x 16,
// so the block tile is BM = 16 WM TM rows by BN = 16 WN TN columns, chosen per
// shape so that the tile count matches the 256 compute units (e.g. 256 x 224 for
// N = 6912, 256 x 80 for N = 2560).  K advances 64 per step:
//  * the A (q) tile BM x 64 int8 is copied to LDS as it is;
//  * the B tile is loaded packed (16 bytes per row and step) and expanded once per
//    workgroup to the signed ternary weights t = c - 1 as int8, in k order, in LDS
//    (ternary4: 5 VALU ops per 4 weights);
//  * LDS is double-buffered: the global loads of step s + 1 are in flight while
//    the MFMAs of step s run; one barrier per step.  Where nearly every thread has a
//    B piece (the 256 x 224 tile) the step is one branch-free basic block whose
//    instruction order is set with scheduling groups: MFMAs interleaved with the
//    next substep's fragment reads, then with the B expansion and the LDS stores
//    (up shape 55.2 -> 52-54 us);
//  * both operands assign the same k to the same (lane, byte) position, which is
//    all the MFMA needs: the sum over k is order-free in integers;
//  * epilogue: y = fp32(acc * c_m), c_m = (s_x[m] * s_w) / 127 in float64; an
//    output without the int32 accumulators goes through LDS so that each store
//    covers whole row segments (fp32 up shape at M = 2048: 59.1 -> 54.5 us).
#include "device_common.h"
#include "internal.h"

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u_g __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u_g gv4u_g;

#ifndef BITNET_GEMM_SCHED
#define BITNET_GEMM_SCHED 1
#endif
#ifndef BITNET_GEMM_SCHED_VALU
#define BITNET_GEMM_SCHED_VALU 2
#endif
#ifndef BITNET_GEMM_SCHED_WR
#define BITNET_GEMM_SCHED_WR 2
#endif
#ifndef BITNET_GEMM_GROUP_M
#define BITNET_GEMM_GROUP_M 2
#endif
// tile configurations 0 (256 x 224) and 1 (256 x 80): waves M, waves N, MFMA
// tiles per wave in M and N, 64-k substeps per barrier step
#ifndef BITNET_GEMM_CFG0
#define BITNET_GEMM_CFG0 4, 2, 4, 7, 2
#endif
#ifndef BITNET_GEMM_CFG0_K64
#define BITNET_GEMM_CFG0_K64 4, 2, 4, 7, 1
#endif
#ifndef BITNET_GEMM_CFG1
#define BITNET_GEMM_CFG1 8, 1, 2, 5, 2
#endif
#ifndef BITNET_GEMM_CFG1_K64
#define BITNET_GEMM_CFG1_K64 8, 1, 2, 5, 1
#endif

// The output tile is written once and never read back here: fp32 values go out as
// non-temporal stores (down shape 70.9 -> 69.1 us at M = 2048); 2-byte bf16 ones
// stay ordinary stores (non-temporal, they were slower: 60.5 -> 66.5 us on up).
__device__ __forceinline__ void store_y_stream(const OutSpec &out, size_t o, double v) {
    if (out.bf16) store_y(out, o, v);
    else __builtin_nontemporal_store((float)v, reinterpret_cast<float *>(out.y) + o);
}

// The 4 weights of one packed byte (k = 4j + i in bits 2i..2i+1) as 4 signed int8
// t = c - 1 in k order: spread the byte so that byte i of a dword holds code i in
// its low two bits, then map each code through a 4-entry byte table with one byte
// permute (0 -> -1, 1 -> 0, 2 -> +1, 3 -> +2).
__device__ __forceinline__ uint32_t ternary4(uint32_t byte) {
    uint32_t sp = byte | (byte << 6);
    sp = (sp | (sp << 12)) & 0x03030303u;
    return __builtin_amdgcn_perm(0u, 0x020100FFu, sp);
}

// 16 packed weights (one dword) as 16 int8 weights in k order.
__device__ __forceinline__ uint4 ternary16(uint32_t w) {
    return make_uint4(ternary4(w & 0xFFu), ternary4((w >> 8) & 0xFFu), ternary4((w >> 16) & 0xFFu), ternary4(w >> 24));
}

__device__ __forceinline__ uint4 gld16(const void *p) {
    const v4u_g v = *(gv4u_g *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int WM, int WN, int TM, int TN, int KS>
__global__ __launch_bounds__(64 * WM * WN, WM * WN <= 4 ? 2 : 1) void gemm_kernel(const int8_t *__restrict__ q,
                                                           const float *__restrict__ s_x,
                                                           const uint8_t *__restrict__ packed,
                                                           const float *__restrict__ s_w, int M, int N,
                                                           int K, const OutSpec out,
                                                           int32_t *__restrict__ acc_out, int tiles_m,
                                                           int tiles_n) {
    constexpr int NT = 64 * WM * WN;          // threads
    constexpr int BM = 16 * WM * TM, BN = 16 * WN * TN;
    constexpr int BK = 64 * KS;               // k per barrier step
    constexpr int RS = BK + 16;               // LDS row stride (bytes): +16 keeps b128 reads conflict-free
    constexpr int CPR = BK / 16;              // 16-byte pieces per A row and step
    constexpr int A_PIECES = BM * CPR;
    constexpr int A_PER_T = (A_PIECES + NT - 1) / NT;
    constexpr int B_PIECES = BN * KS;         // 16-byte packed pieces per step
    constexpr int B_PER_T = (B_PIECES + NT - 1) / NT;
    // Clamped, branch-free staging (see load_step) only where nearly every thread has
    // a B piece: elsewhere the repeated pieces cost more VALU and LDS time than the
    // interleaving gains (256 x 80 tile: 65 -> 70 us on the down shape).
    constexpr bool CLAMP = (B_PIECES % NT == 0) || 8 * (B_PIECES % NT) >= 7 * NT;
    // A and B staging share one allocation, reused after the k loop to stage the
    // fp32 output rows (row stride CWP floats: +4 spreads a lane group's 4 rows over
    // distinct banks)
    constexpr int A_BYTES = 2 * BM * RS, B_BYTES = 2 * BN * RS;
    constexpr int CW = 16 * TN, CWP = CW + 4;
    static_assert(WM * WN * 16 * CWP * 4 <= A_BYTES + B_BYTES, "output staging exceeds LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[A_BYTES + B_BYTES];
    uint8_t (*As)[BM * RS] = reinterpret_cast<uint8_t (*)[BM * RS]>(smem);
    uint8_t (*Bs)[BN * RS] = reinterpret_cast<uint8_t (*)[BN * RS]>(smem + A_BYTES);
    __shared__ double rowscale[BM];

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; give each
    // XCD a contiguous range of tiles, column-major in groups of GM M tiles, so that
    // workgroups sharing A rows and B columns share that XCD's L2 (GM = 2: an XCD's
    // share of A and B for the up shape is about 3.5 MB of its 4 MB L2).
    const int nt = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int q8 = nt / 8, r8 = nt % 8, x = bid % 8;
    const int t = x * q8 + min(x, r8) + bid / 8;
    const int GM = BITNET_GEMM_GROUP_M;
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsize = min(GM, tiles_m - first_m);
    const int tm = first_m + (t % (GM * tiles_n)) % gsize;
    const int tn = (t % (GM * tiles_n)) / gsize;
    const int m_base = tm * BM, n_base = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int KB = K >> 2;
    const int steps = K / BK;                 // K % BK == 0 (checked by the launcher)

    // staging: A piece p = tid + NT * i -> row p / CPR, piece p % CPR (CPR
    // consecutive threads cover a row's BK bytes); B piece p -> row p / KS, part p % KS.

    // With CLAMP, piece indices and rows are clamped instead of guarded, so that the
    // loop body is one basic block the scheduler can interleave: threads past the
    // last piece repeat it (same bytes to the same LDS address), A rows past M repeat
    // row M - 1 and B rows past N repeat row N - 1 (they only feed outputs that are
    // never stored).  Without it, missing pieces are skipped and rows past the end
    // load zeros.
    uint4 ra[A_PER_T], rb[B_PER_T];
    auto load_step = [&](int s) {
        const int k0 = s * BK;
        #pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int p = CLAMP ? min(tid + NT * i, A_PIECES - 1) : tid + NT * i;
            const int row = p / CPR, ch = p % CPR;
            const int gm = m_base + row;
            if (CLAMP) ra[i] = gld16(q + (size_t)min(gm, M - 1) * K + k0 + 16 * ch);
            else ra[i] = (p < A_PIECES && gm < M) ? gld16(q + (size_t)gm * K + k0 + 16 * ch) : make_uint4(0u, 0u, 0u, 0u);
        }
        #pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int p = CLAMP ? min(tid + NT * i, B_PIECES - 1) : tid + NT * i;
            const int r = p / KS, part = p % KS;
            const int gn = n_base + r;
            if (CLAMP) rb[i] = gld16(packed + (size_t)min(gn, N - 1) * KB + (k0 >> 2) + 16 * part);
            else rb[i] = (p < B_PIECES && gn < N) ? gld16(packed + (size_t)gn * KB + (k0 >> 2) + 16 * part)
                                                  : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_step = [&](int buf) {
        #pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int p = CLAMP ? min(tid + NT * i, A_PIECES - 1) : tid + NT * i;
            if (CLAMP || p < A_PIECES) {
                const int row = p / CPR, ch = p % CPR;
                *reinterpret_cast<uint4 *>(&As[buf][row * RS + 16 * ch]) = ra[i];
            }
        }
        #pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int p = CLAMP ? min(tid + NT * i, B_PIECES - 1) : tid + NT * i;
            if (CLAMP || p < B_PIECES) {
                const int r = p / KS, part = p % KS;
                const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
                #pragma unroll
                for (int d = 0; d < 4; ++d)
                    *reinterpret_cast<uint4 *>(&Bs[buf][r * RS + 64 * part + 16 * d]) = ternary16(w[d]);
            }
        }
    };

    v4i acc[TM][TN];
    #pragma unroll
    for (int i = 0; i < TM; ++i)
        #pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int l16 = lane & 15, g = lane >> 4;
    load_step(0);
    store_step(0);
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        // with CLAMP the last step reloads and restages its own tile into the idle
        // buffer (never read), which keeps the body free of branches
        if (CLAMP) load_step(min(s + 1, steps - 1));
        else if (s + 1 < steps) load_step(s + 1);
        #pragma unroll
        for (int u = 0; u < KS; ++u) {
            v4i a[TM], b[TN];
            #pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = *reinterpret_cast<const v4i *>(&As[buf][(wm * TM * 16 + i * 16 + l16) * RS + 64 * u + 16 * g]);
            #pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = *reinterpret_cast<const v4i *>(&Bs[buf][(wn * TN * 16 + j * 16 + l16) * RS + 64 * u + 16 * g]);
            #pragma unroll
            for (int i = 0; i < TM; ++i)
                #pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (CLAMP || s + 1 < steps) store_step(buf ^ 1);
#if BITNET_GEMM_SCHED
        // Instruction order within the step: the global loads first, the first
        // substep's fragment reads, then the MFMAs with the next substep's fragment
        // reads between them, and in the last substep the B expansion (VALU) and the
        // LDS stores of the next step between the MFMAs.
        if (CLAMP) {
            constexpr int NMF = TM * TN, NRD = TM + TN, NWR = A_PER_T + 4 * B_PER_T;
            __builtin_amdgcn_sched_group_barrier(0x020, A_PER_T + B_PER_T, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
            #pragma unroll
            for (int u = 0; u < KS; ++u) {
                #pragma unroll
                for (int m = 0; m < NMF; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (u + 1 < KS) {
                        if (m < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    } else {
                        __builtin_amdgcn_sched_group_barrier(0x002, BITNET_GEMM_SCHED_VALU, 0);
                        if (m % BITNET_GEMM_SCHED_WR == BITNET_GEMM_SCHED_WR - 1 && m / BITNET_GEMM_SCHED_WR < NWR)
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    }
                }
            }
        }
#endif
        __syncthreads();
    }

    // per-row rescale factors
    const float sw = *s_w;
    for (int row = tid; row < BM; row += NT) {
        const int gm = m_base + row;
        rowscale[row] = gm < M ? rescale_factor(s_x[gm], sw) : 0.0;
    }
    __syncthreads();

    // 16x16 accumulator layout: lane -> column l16; register r -> row 4 * (lane / 16) + r.
    // The bias of the lane's TN columns is loaded once, before any store.
    float bcol[TN];
    #pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n_base + wn * TN * 16 + j * 16 + l16;
        bcol[j] = (out.bias && col < N) ? out.bias[col] : 0.0f;
    }
    if (!acc_out) {
        // Output without the int32 accumulators: each wavefront writes its rescaled
        // 16 x CW fp32 block of one M tile to LDS, then stores whole row segments
        // (consecutive lanes on consecutive 4-column chunks) instead of pieces of 4
        // rows x 16 columns per instruction; bf16 outputs are rounded from the same
        // fp32 values on the way out.
        float *stage = reinterpret_cast<float *>(smem) + wave * 16 * CWP;
        const int col0 = n_base + wn * TN * 16;
        const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(out.y) & (out.bf16 ? 7 : 15)) == 0;
        #pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row0 = m_base + wm * TM * 16 + i * 16;
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lr = wm * TM * 16 + i * 16 + 4 * g + r;
                const int row = m_base + lr;
                const double cm = rowscale[lr];
                const float sxr = (out.w_group && row < M) ? s_x[row] : 0.0f;
                #pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = col0 + j * 16 + l16;
                    double yv = 0.0;
                    if (row < M && col < N) {
                        yv = (double)acc[i][j][r] * col_factor(out, s_w, col, sxr, cm);
                        if (out.bias) yv += (double)bcol[j];
                    }
                    stage[(4 * g + r) * CWP + j * 16 + l16] = (float)yv;
                }
            }
            __syncthreads();
            constexpr int CH = 16 * (CW / 4);     // 4-column chunks in the block
            #pragma unroll
            for (int c = lane; c < CH; c += 64) {
                const int rr = c / (CW / 4), cc = 4 * (c % (CW / 4));
                const int row = row0 + rr, col = col0 + cc;
                if (row >= M || col >= N) continue;
                const v4f v = *reinterpret_cast<const v4f *>(&stage[rr * CWP + cc]);
                const size_t o = (size_t)row * N + col;
                if (out.bf16) {
                    uint16_t *dst = reinterpret_cast<uint16_t *>(out.y) + o;
                    const uint16_t h[4] = {bf16_rne(v.x), bf16_rne(v.y), bf16_rne(v.z), bf16_rne(v.w)};
                    if (vec) {
                        *reinterpret_cast<uint2 *>(dst) = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                                    (uint32_t)h[2] | ((uint32_t)h[3] << 16));
                    } else {
                        for (int d = 0; d < 4 && col + d < N; ++d) dst[d] = h[d];
                    }
                } else {
                    float *dst = reinterpret_cast<float *>(out.y) + o;
                    if (vec) {
                        __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(dst));
                    } else {
                        const float e[4] = {v.x, v.y, v.z, v.w};
                        for (int d = 0; d < 4 && col + d < N; ++d) __builtin_nontemporal_store(e[d], dst + d);
                    }
                }
            }
            __syncthreads();
        }
        return;
    }
    #pragma unroll
    for (int i = 0; i < TM; ++i) {
        #pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lr = wm * TM * 16 + i * 16 + 4 * g + r;
            const int row = m_base + lr;
            if (row >= M) continue;
            const double cm = rowscale[lr];
            const float sxr = out.w_group ? s_x[row] : 0.0f;
            #pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n_base + wn * TN * 16 + j * 16 + l16;
                if (col < N) {
                    const size_t o = (size_t)row * N + col;
                    const int v = acc[i][j][r];
                    double yv = (double)v * col_factor(out, s_w, col, sxr, cm);
                    if (out.bias) yv += (double)bcol[j];
                    store_y_stream(out, o, yv);
                    if (acc_out) acc_out[o] = v;
                }
            }
        }
    }
}

struct GemmCfg { int wm, wn, tm, tn; };

template <int WM, int WN, int TM, int TN, int KS>
static hipError_t launch_cfg(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                             int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    constexpr int BM = 16 * WM * TM, BN = 16 * WN * TN;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    gemm_kernel<WM, WN, TM, TN, KS><<<dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * WM * WN), 0, st>>>(
        q, s_x, packed, s_w, (int)M, (int)N, (int)K, y, acc, tiles_m, tiles_n);
    return hipGetLastError();
}

// Tile configurations (id: BM x BN): 0: 256 x 224, 1: 256 x 80, 2: 256 x 128,
// 3: 128 x 128, 4: 64 x 128.  Pick the tile whose busiest compute unit does the least
// work, assuming one workgroup per CU at a time: cost = ceil(tiles / 256) * BM * BN.
static int gemm_pick(int64_t M, int64_t N, int64_t *tiles_out) {
    struct Cand { int bm, bn, id; };
    const Cand cands[] = {{256, 224, 0}, {256, 80, 1}, {256, 128, 2}, {128, 128, 3}, {64, 128, 4}};
    int best = 3;
    int64_t best_cost = -1, best_tiles = 0;
    for (const Cand &c : cands) {
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        const int64_t cost = ((tiles + 255) / 256) * (int64_t)c.bm * c.bn;
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = c.id; best_tiles = tiles; }
    }
    if (tiles_out) *tiles_out = best_tiles;
    return best;
}

// The pipelined kernel (gemm_pipe.hip) where its whole 128-weight steps fit, except
// where this file's 256 x 224 tile covers the problem in one round and the pipelined
// kernel needs two or more (M = 2048, N = 6912, K = 2560: 47.6 against 50.0 us;
// M = 1024, N = 13824: 49.8 against 53.3 us).  Elsewhere it measured faster at every
// M = 512 .. 4096, N = 640 .. 13824, K = 2560 .. 8192 tried (by 1.03 .. 1.9x).
static bool gemm_use_pipe(int64_t M, int64_t N, int64_t K) {
    if (!gemm_pipe_ok(M, N, K)) return false;
    int64_t tiles = 0;
    const int cfg = gemm_pick(M, N, &tiles);
    return !(cfg == 0 && tiles <= 256 && gemm_pipe_rounds(M, N) >= 2);
}

// Estimated time (us) of launch_gemm.  This file's kernel: rounds of tiles over the
// 256 CUs x K / 64 steps of about 0.55 us, plus about 6 us of launch, prologue and
// epilogue (measured on M = 16 .. 256 against six shapes from 2560 x 2560 to
// 8192 x 28672).
double gemm_estimate_us(int64_t M, int64_t N, int64_t K) {
    if (gemm_use_pipe(M, N, K)) return gemm_pipe_estimate_us(M, N, K);
    int64_t tiles = 0;
    gemm_pick(M, N, &tiles);
    return (double)((tiles + 255) / 256) * (double)(K / 64) * 0.55 + 6.0;
}

hipError_t launch_gemm(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                       int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    // group-wise scales: the pipelined kernel only
    if (gemm_use_pipe(M, N, K) || (y.w_group > 0 && y.w_group < K)) return launch_gemm_pipe(0, q, s_x, packed, s_w, M, N, K, y, acc, st);
    return launch_gemm_cfg(gemm_pick(M, N, nullptr), q, s_x, packed, s_w, M, N, K, y, acc, st);
}

// configurations 0..4: this file's tiles; 5, 6: the pipelined kernel with 128 x 224
// and 128 x 160 tiles
int gemm_config_count() { return 7; }

hipError_t launch_gemm_cfg(int cfg, const int8_t *q, const float *s_x, const uint8_t *packed,
                           const float *s_w, int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc,
                           hipStream_t st) {
    // a configuration needing K % 128 == 0 falls back to its single-step twin
    const bool k128 = (K % 128) == 0;
    switch (cfg) {
        case 0: return k128 ? launch_cfg<BITNET_GEMM_CFG0>(q, s_x, packed, s_w, M, N, K, y, acc, st)
                            : launch_cfg<BITNET_GEMM_CFG0_K64>(q, s_x, packed, s_w, M, N, K, y, acc, st);
        case 1: return k128 ? launch_cfg<BITNET_GEMM_CFG1>(q, s_x, packed, s_w, M, N, K, y, acc, st)
                            : launch_cfg<BITNET_GEMM_CFG1_K64>(q, s_x, packed, s_w, M, N, K, y, acc, st);
        case 5:
        case 6:
            // the pipelined kernel where its whole 128-weight steps fit, else the
            // matching tile of this file
            if (gemm_pipe_ok(M, N, K)) return launch_gemm_pipe(cfg == 5 ? 7 : 5, q, s_x, packed, s_w, M, N, K, y, acc, st);
            return launch_gemm_cfg(cfg - 5, q, s_x, packed, s_w, M, N, K, y, acc, st);
        case 2: return launch_cfg<2, 2, 8, 4, 1>(q, s_x, packed, s_w, M, N, K, y, acc, st);
        case 3: return launch_cfg<2, 2, 4, 4, 1>(q, s_x, packed, s_w, M, N, K, y, acc, st);
        default: return launch_cfg<1, 4, 4, 2, 1>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    }
}

}  // namespace bitnet
