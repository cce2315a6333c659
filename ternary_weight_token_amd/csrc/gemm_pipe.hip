// Prefill GEMM, pipelined and persistent: the contraction and rescale of the
// BitLinear forward (pages: chenxutan.com sec. 2.3 rescale, sec. 3.1
// BitLinear.forward over the quantized operands) as int8 x ternary -> int32 on
// the matrix cores (v_mfma_i32_16x16x64_i8), for many tokens.
//
// Workgroup: 8 wavefronts, two per SIMD, with two roles; output tile 128 x BN,
// BN = 32 TN weight rows; one k-step is 128 weights.
//  * 4 producer waves load the step's q rows (whole 128-byte lines) and packed
//    weight rows (32 bytes each; 64 bytes per pair of steps where K is a multiple
//    of 256) into registers three steps ahead, and write them to one of three LDS
//    stages: the q bytes of each 16-byte chunk in the
//    transposed order k = 4d + i -> byte 4i + d (four byte permutes per dword),
//    chunks XOR-swizzled so that fragment reads are free of bank conflicts.
//  * 4 consumer waves (2 x 2), each 64 token rows x 16 TN weight rows: read the
//    q fragments and one packed dword per weight fragment, and turn the dword
//    into the MFMA operand with one shift and one mask per 4 codes: dword i of
//    the operand holds code i of each packed byte, which is the same transposed
//    k order as the q bytes.  The products run on the codes c; sum q (c - 1) =
//    sum q c - sum q, the row sums of q gathered from the q fragments with
//    byte dot products.  At the end of a tile each consumer rescales and stores
//    its block straight from the accumulators (y = fp32(acc c_m), c_m = (s_x s_w)
//    / 127 in float64; the weights are the MFMA's first operand, so a lane holds
//    4 consecutive output columns of one token row: one 16-byte store).
// Expanding the codes in registers keeps LDS traffic to the staged bytes (LDS
// writes run at about a quarter of the read rate here).
//
// The grid is one workgroup per compute unit; workgroup b takes tiles b, b + G,
// ... in column-major order of M tiles.  The step sequence runs across tile
// boundaries, loads for the next tile starting while the current one computes;
// the k order is rotated per workgroup (the sum over k is order-free), so that
// workgroups reading the same rows are at different k at any moment.
#include "device_common.h"
#include "internal.h"

#ifndef BITNET_PIPE_SGN
#define BITNET_PIPE_SGN 1   // group-wise scales, groups up to 128: signed operands
#endif

namespace bitnet {

namespace {

typedef int pv4i __attribute__((ext_vector_type(4)));
typedef float pv4f __attribute__((ext_vector_type(4)));
typedef unsigned int pv4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const pv4u gpv4u;

constexpr int kPipeBM = 128;                    // token rows per tile (2 consumer waves x 64)
constexpr int kPipeKS = 128;                    // weights per k-step (one 128-byte line of q per row)
constexpr int kPipeA = kPipeBM * kPipeKS;       // q bytes per stage
constexpr int kPipeBp = 256 * 32;               // packed weight bytes per stage (up to 256 rows)
constexpr int kPipeBp2 = 256 * 64;              // the same for a pair of steps (PW)
constexpr int kPipeD = 3;                       // stages
constexpr int kPipeThreads = 512;

__device__ __forceinline__ pv4u gload(const void *p) { return *(gpv4u *)p; }

// LDS slot of 16-byte chunk c (0..7) of local q row r within its 128-byte row:
// the chunk index XORed with the row's position, so that the 16 lanes of a
// fragment read (16 rows, one chunk) hit distinct banks.
__device__ __forceinline__ int qslot(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

}  // namespace

// TN: 16-row weight blocks per consumer wave (tile BN = 32 TN).
// OPT: the epilogue options (bias, bf16 output, one weight scale per output
// channel) are compiled in; without them the store path is fp32 y (and acc).
// GRP: group-wise weight scales (out.w_group = G < K, G = 64 or a multiple of 128):
// the int32 products of each group are scaled into fp32 accumulators when the
// group's last half step is done (see the consumer); OPT is set as well.
// SGN (GRP with groups of at most 128 weights, a fold every step or half step): the
// codes are expanded to the signed weights t = c - 1 (one byte permute per dword,
// code 3 as +2), so that each group's products are sum q t itself and the fold has no
// sum of q to subtract; the same integers, so the same results.
// PW (K a multiple of 256): the packed weights of a pair of steps (k-steps 2j and
// 2j + 1) are loaded together as 64-byte row pieces on the even step and staged in
// its stage; the odd step reads them from there.  A load instruction then covers 16
// rows in 64-byte pieces instead of 32 rows in 32-byte pieces: half the cache lines
// per staged byte.
template <int TN, bool OPT, bool GRP = false, bool PW = false, bool SGN = false>
__global__ __launch_bounds__(kPipeThreads, 1) void gemm_pipe_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s_x, const uint8_t *__restrict__ packed,
    const float *__restrict__ s_w, int M, int N, int K, const OutSpec out, int32_t *__restrict__ acc_out,
    int tiles_m, int n_tiles) {
    constexpr int BN = 32 * TN;
    static_assert(BN <= 256, "packed stage holds 256 rows");
    constexpr int D = kPipeD;
    constexpr int Stage = kPipeA + (PW ? kPipeBp2 : kPipeBp);
    __shared__ __attribute__((aligned(1024))) uint8_t smem[D * Stage];
    // per tile (4 slots, tile index % 4): sum over k of q for each of the 128 rows
    __shared__ int sqbuf[4][kPipeBM];
    // GRP, per stage: sum of q over each half step (64 weights) of the 128 rows, and
    // the weight scale of each half step's group for the BN rows
    __shared__ int sqh[GRP ? D : 1][2][kPipeBM];
    __shared__ __attribute__((aligned(16))) float scs[GRP ? D : 1][2][BN];

    // the wave index is the same in every lane: keep it (and what derives from it) scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, wg = blockIdx.x;
    const int my_tiles = (n_tiles - wg + G - 1) / G;
    const int KS = K / kPipeKS;
    const int total = my_tiles * KS;
    const size_t KB = (size_t)(K >> 2);
    // k order rotated per workgroup: workgroups that share q rows (one XCD, one M
    // tile) or weight rows (one N tile) start at different k; GRP: at a group start,
    // so that every group's half steps follow one another
    const int gh = GRP ? out.w_group / 64 : 1;    // half steps per group
    const int ng = GRP ? K / out.w_group : 1;
    // (PW: at an even step, so that the pairs are k-steps 2j, 2j + 1)
    int kr0;
    {
        const int kx = wg & 7, kj = wg >> 3, kjn = (G + 7) >> 3;
        kr0 = (int)(((int64_t)kj * KS / kjn + 3 * kx) % KS);
        int al = (GRP && gh > 2) ? gh / 2 : 1;
        if (PW && (al & 1)) al *= 2;
        kr0 -= kr0 % al;
    }

    if (wave >= 4) {
        // ------------------------------------------------------------ producer
        const int tp = tid - 256;
        constexpr int NB = (2 * BN + 255) / 256;          // packed chunks per thread (1 or 2)
        // chunks of this thread: q chunk tp + 256 h -> row (tp >> 3) + 32 h, 16-byte
        // chunk tp & 7 (eight lanes per 128-byte line); packed chunk tp + 256 h ->
        // row (tp >> 1) + 128 h, half tp & 1
        const int ar = tp >> 3, ac = tp & 7, br = tp >> 1, bh = tp & 1;
        // packed chunks past the tile's rows: the last waves have none in the
        // second slot (a wave-uniform condition)
        const bool b2 = NB > 1 && 256 + tp < 2 * BN;
        // PW: piece wc of the pair's 64 bytes of rows wr + 64 h; the rows past the
        // tile's BN (a multiple of 32) fall on whole waves
        constexpr int NW = PW ? (BN + 63) / 64 : 2;
        const int wr = tp >> 2, wc = tp & 3;
        int d_s = 0, d_ti = 0, d_kk = 0;
        int d_kr = kr0;
        const int8_t *arow[4];
        const uint8_t *brow[NW];
        int bn0 = 0;   // first weight row of the tile being loaded
        auto set_tile = [&](int ti) {
            const int t = wg + ti * G;
            const int m0 = (t % tiles_m) * kPipeBM, n0 = (t / tiles_m) * BN;
            bn0 = n0;
            #pragma unroll
            for (int h = 0; h < 4; ++h) arow[h] = q + (size_t)min(m0 + ar + 32 * h, M - 1) * K + 16 * ac;
            if (PW) {
                #pragma unroll
                for (int h = 0; h < NW; ++h) brow[h] = packed + (size_t)min(n0 + wr + 64 * h, N - 1) * KB + 16 * wc;
            } else {
                #pragma unroll
                for (int h = 0; h < 2; ++h) brow[h] = packed + (size_t)min(n0 + br + 128 * h, N - 1) * KB + 16 * bh;
            }
        };
        set_tile(0);
        // loads of step d_s (clamped to the last step) into register set R
        // (PW: only the even sets hold weights, the pair's pieces)
        pv4u ra[4][4], rb[4][NW];
        // GRP: scale entries tp and tp + 256 of the step's 2 x BN (half, row) pairs
        float rsc[GRP ? 4 : 1][2];
        auto issue = [&](int R) {
            #pragma unroll
            for (int h = 0; h < 4; ++h) ra[R][h] = gload(arow[h] + (size_t)d_kr * kPipeKS);
            if (PW) {
                // the set's parity is the step's; past the last step d_kr stays at
                // an odd k-step, whose pair starts one step earlier
                if ((R & 1) == 0) {
                    #pragma unroll
                    for (int h = 0; h < NW; ++h)
                        if (64 * h + wr < BN) rb[R][h] = gload(brow[h] + (size_t)(d_kr & ~1) * (kPipeKS / 4));
                }
            } else {
                rb[R][0] = gload(brow[0] + (size_t)d_kr * (kPipeKS / 4));
                if (b2) rb[R][1] = gload(brow[1] + (size_t)d_kr * (kPipeKS / 4));
            }
            if (GRP) {
                #pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    const int e = tp + 256 * e2;   // e2 = 1: whole waves with or without an entry
                    if (e < 2 * BN) {
                        const int u = e >= BN ? 1 : 0, c = e - u * BN;
                        rsc[R][e2] = s_w[(size_t)min(bn0 + c, N - 1) * ng + (2 * d_kr + u) / gh];
                    }
                }
            }
            ++d_s;
            if (d_s < total) {
                if (++d_kr == KS) d_kr = 0;
                if (++d_kk == KS) {
                    d_kk = 0;
                    set_tile(++d_ti);
                }
            }
        };
        // row sums of q over the tile, this thread's chunk of rows ar + 32 h
        int psq[4] = {0, 0, 0, 0};
        int t_ti = 0, t_kk = 0;   // tile and k-step of the step being stored
        // register set R (step x) into stage x % 3: q chunks transposed and
        // swizzled, packed halves swapped on rows with bit 3 set
        auto store = [&](int x, int R) {
            uint8_t *st = smem + (x % D) * Stage;
            #pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int r = ar + 32 * h;
                int t = __builtin_amdgcn_sdot4((int)ra[R][h].x, 0x01010101, GRP ? 0 : psq[h], false);
                t = __builtin_amdgcn_sdot4((int)ra[R][h].y, 0x01010101, t, false);
                t = __builtin_amdgcn_sdot4((int)ra[R][h].z, 0x01010101, t, false);
                t = __builtin_amdgcn_sdot4((int)ra[R][h].w, 0x01010101, t, false);
                if (GRP) {
                    // the half step's sum of q for row r: chunks ac & ~3 .. + 3
                    t += __shfl_xor(t, 1, 64);
                    t += __shfl_xor(t, 2, 64);
                    if ((ac & 3) == 0) sqh[x % D][ac >> 2][r] = t;
                } else {
                    psq[h] = t;
                }
                uint32_t p0, p1, p2, p3;
                transpose4x4(ra[R][h].x, ra[R][h].y, ra[R][h].z, ra[R][h].w, p0, p1, p2, p3);
                *reinterpret_cast<uint4 *>(st + 1024 * (r >> 3) + 128 * (r & 7) + 16 * qslot(r, ac)) =
                    make_uint4(p0, p1, p2, p3);
            }
            if (PW) {
                // 64 bytes per row, the 16-byte pieces XOR-swizzled by bits 2..3 of
                // the row: the consumers' 16 rows of a fragment read hit distinct banks
                if ((R & 1) == 0) {
                    #pragma unroll
                    for (int h = 0; h < NW; ++h) {
                        const int r = wr + 64 * h;
                        if (r < BN) *reinterpret_cast<pv4u *>(st + kPipeA + 64 * r + 16 * (wc ^ ((r >> 2) & 3))) = rb[R][h];
                    }
                }
            } else {
                #pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (h == 0 || b2) {
                        const int r = br + 128 * h;
                        *reinterpret_cast<pv4u *>(st + kPipeA + 32 * r + 16 * (bh ^ ((r >> 3) & 1))) = rb[R][h];
                    }
                }
            }
            if (GRP) {
                #pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    const int e = tp + 256 * e2;
                    if (e < 2 * BN) (&scs[x % D][0][0])[e] = rsc[R][e2];
                }
            }
            // the tile's last step: each row's sum over its eight chunk lanes, into
            // the tile's slot (read by the consumers after two more barriers)
            if (!GRP && x < total && ++t_kk == KS) {
                #pragma unroll
                for (int h = 0; h < 4; ++h) {
                    int v = psq[h];
                    v += __shfl_xor(v, 1, 64);
                    v += __shfl_xor(v, 2, 64);
                    v += __shfl_xor(v, 4, 64);
                    if (ac == 0) sqbuf[t_ti & 3][ar + 32 * h] = v;
                    psq[h] = 0;
                }
                t_kk = 0;
                ++t_ti;
            }
        };
        // register set of step x: x % 4
        issue(0);
        issue(1);
        issue(2);
        issue(3);
        store(0, 0);
        issue(0);
        store(1, 1);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // iteration s: loads of step s + 5 into the set of step s + 1 (stored in the
        // last iteration), step s + 2 from its set into the stage of step s - 1 (read
        // up to the last barrier); three steps of loads stay in flight
        auto body = [&](int s, int Ri, int Rs) {
            issue(Ri);
            store(s + 2, Rs);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        };
        int s = 0;
        for (; s + 4 <= total; s += 4) {
            body(s, 1, 2);
            body(s + 1, 2, 3);
            body(s + 2, 3, 0);
            body(s + 3, 0, 1);
        }
        if (s < total) body(s, 1, 2);
        if (s + 1 < total) body(s + 1, 2, 3);
        if (s + 2 < total) body(s + 2, 3, 0);
        return;
    }

    // ---------------------------------------------------------------- consumer
    const int l16 = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    pv4i acc[4][TN];
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        #pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = pv4i{0, 0, 0, 0};
    // GRP: sum over groups of (acc_g - sum_g q) s_g in fp32, the running sum of q of
    // the current group per row, and the half steps of the group done so far
    pv4f facc[GRP ? 4 : 1][GRP ? TN : 1];
    int sqrun[4] = {0, 0, 0, 0};
    int c_h = 0;
    if (GRP) {
        #pragma unroll
        for (int i = 0; i < 4; ++i)
            #pragma unroll
            for (int j = 0; j < TN; ++j) facc[i][j] = pv4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // per-lane offsets: the q fragment of half u (local row r = 64 wm + 16 i + l16
    // lies in 1 KB block r / 8 at position r % 8 = lane % 8, chunk 4u + g at its
    // slot) and the packed dword 4u + g of weight row r (halves swapped on rows with
    // bit 3 set: dword 4u + g sits at (4u + g) ^ 4)
    // (PW: dword g of piece 2 (x & 1) + u of the pair's 64 bytes, swizzled as stored)
    int aoff[2], boff[2];
    #pragma unroll
    for (int u = 0; u < 2; ++u) {
        aoff[u] = 1024 * (8 * wm + ((lane >> 3) & 1)) + 128 * (lane & 7) + 16 * qslot(lane & 15, 4 * u + g);
        boff[u] = kPipeA + 32 * (16 * TN * wn + l16) + 4 * ((4 * u + g) ^ (4 * ((l16 >> 3) & 1)));
    }
    const int pwoff = kPipeA + 64 * (16 * TN * wn + l16) + 4 * g, pwsw = (l16 >> 2) & 3;
    pv4i fa[2][4];
    uint32_t fb[2][TN];
    auto read = [&](int x, int u) {
        const uint8_t *st = smem + (x % D) * Stage;
        #pragma unroll
        for (int i = 0; i < 4; ++i) fa[u][i] = *reinterpret_cast<const pv4i *>(st + aoff[u] + 2048 * i);
        if (PW) {
            const uint8_t *sb = smem + ((x & ~1) % D) * Stage + pwoff + 16 * ((2 * (x & 1) + u) ^ pwsw);
            #pragma unroll
            for (int j = 0; j < TN; ++j) fb[u][j] = *reinterpret_cast<const uint32_t *>(sb + 1024 * j);
        } else {
            #pragma unroll
            for (int j = 0; j < TN; ++j) fb[u][j] = *reinterpret_cast<const uint32_t *>(st + boff[u] + 512 * j);
        }
    };
    auto half = [&](int u) {
        #pragma unroll
        for (int j = 0; j < TN; ++j) {
            // dword i of the operand: code i of each packed byte (k = 4d + i at byte 4i + d)
            const uint32_t w = fb[u][j];
            pv4i b{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
                   (int)((w >> 6) & 0x03030303u)};
            if (SGN) {
                #pragma unroll
                for (int d = 0; d < 4; ++d) b[d] = (int)__builtin_amdgcn_perm(0u, 0x020100FFu, (uint32_t)b[d]);
            }
            #pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, fa[u][i], acc[i][j], 0, 0, 0);
        }
    };
    // GRP, after half u of step x: at the group's last half, its products (codes c,
    // less the group's sum of q; SGN: the signed weights) times the group scale of
    // each column into facc
    auto fold_half = [&](int x, int u) {
        const int st = x % D;
        if (!SGN) {
            #pragma unroll
            for (int i = 0; i < 4; ++i) sqrun[i] += sqh[st][u][64 * wm + 16 * i + l16];
        }
        if (++c_h == gh) {
            c_h = 0;
            #pragma unroll
            for (int j = 0; j < TN; ++j) {
                const pv4f s4 = *reinterpret_cast<const pv4f *>(&scs[st][u][16 * TN * wn + 16 * j + 4 * g]);
                #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) facc[i][j][r] += (float)(SGN ? acc[i][j][r] : acc[i][j][r] - sqrun[i]) * s4[r];
                    acc[i][j] = pv4i{0, 0, 0, 0};
                }
            }
            #pragma unroll
            for (int i = 0; i < 4; ++i) sqrun[i] = 0;
        }
    };
    const float sw = GRP ? 0.0f : *s_w;
    int c_ti = 0, c_kk = 0;
    float sxr[4];
    auto load_sx = [&](int ti) {
        const int t = wg + ti * G;
        const int m0 = (t % tiles_m) * kPipeBM + 64 * wm + l16;
        #pragma unroll
        for (int i = 0; i < 4; ++i) sxr[i] = s_x[min(m0 + 16 * i, M - 1)];
    };
    load_sx(0);

    auto epilogue = [&](int ti) {
        const int t = wg + ti * G;
        const int m_base = (t % tiles_m) * kPipeBM + 64 * wm, n_base = (t / tiles_m) * BN + 16 * TN * wn;
        const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(out.y) & (OPT && out.bf16 ? 7 : 15)) == 0 &&
                         (!acc_out || (reinterpret_cast<uintptr_t>(acc_out) & 15) == 0);
        if (vec && m_base + 64 <= M && n_base + 16 * TN <= N && !(OPT && (out.bias || out.w_group || out.bf16))) {
            // whole block inside: one 16-byte store of 4 columns per lane and block
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m_base + 16 * i + l16;
                const double cm = rescale_factor(sxr[i], sw);
                float *yr = reinterpret_cast<float *>(out.y) + (size_t)m * N + n_base + 4 * g;
                #pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const pv4f v{(float)((double)acc[i][j][0] * cm), (float)((double)acc[i][j][1] * cm),
                                 (float)((double)acc[i][j][2] * cm), (float)((double)acc[i][j][3] * cm)};
                    __builtin_nontemporal_store(v, reinterpret_cast<pv4f *>(yr + 16 * j));
                    if (acc_out)
                        *reinterpret_cast<pv4i *>(acc_out + (size_t)m * N + n_base + 4 * g + 16 * j) = acc[i][j];
                }
            }
            return;
        }
        if (OPT && !GRP && vec && m_base + 64 <= M && n_base + 16 * TN <= N && !out.w_group &&
            (reinterpret_cast<uintptr_t>(out.bias) & 15) == 0) {
            // whole block inside with a bias and / or bf16 y (one scale per tensor): the
            // bias of the lane's 4 columns per block read once, before the stores
            pv4f b4[TN];
            #pragma unroll
            for (int j = 0; j < TN; ++j)
                b4[j] = out.bias ? *reinterpret_cast<const pv4f *>(out.bias + n_base + 16 * j + 4 * g)
                                 : pv4f{0.0f, 0.0f, 0.0f, 0.0f};
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m_base + 16 * i + l16;
                const double cm = rescale_factor(sxr[i], sw);
                #pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const size_t o = (size_t)m * N + n_base + 16 * j + 4 * g;
                    float v[4];
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        double yv = (double)acc[i][j][r] * cm;
                        if (out.bias) yv += (double)b4[j][r];
                        v[r] = (float)yv;
                    }
                    if (out.bf16) {
                        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out.y) + o) =
                            make_uint2((uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16),
                                       (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16));
                    } else {
                        __builtin_nontemporal_store(pv4f{v[0], v[1], v[2], v[3]},
                                                    reinterpret_cast<pv4f *>(reinterpret_cast<float *>(out.y) + o));
                    }
                    if (acc_out) *reinterpret_cast<pv4i *>(acc_out + o) = acc[i][j];
                }
            }
            return;
        }
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m_base + 16 * i + l16;
            if (m >= M) continue;
            const double cm = rescale_factor(sxr[i], sw);
            #pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n0 = n_base + 16 * j + 4 * g;
                if (n0 >= N) continue;
                const size_t o = (size_t)m * N + n0;
                float v[4];
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = min(n0 + r, N - 1);
                    double yv;
                    if (GRP) yv = ((double)facc[i][j][r] * (double)sxr[i]) / 127.0;
                    else yv = (double)acc[i][j][r] * ((OPT && out.w_group) ? rescale_factor(sxr[i], s_w[n]) : cm);
                    if (OPT && out.bias) yv += (double)out.bias[n];
                    v[r] = (float)yv;
                }
                if (vec && n0 + 3 < N) {
                    if (OPT && out.bf16) {
                        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out.y) + o) =
                            make_uint2((uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16),
                                       (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16));
                    } else {
                        __builtin_nontemporal_store(pv4f{v[0], v[1], v[2], v[3]},
                                                    reinterpret_cast<pv4f *>(reinterpret_cast<float *>(out.y) + o));
                    }
                    if (acc_out) *reinterpret_cast<pv4i *>(acc_out + o) = acc[i][j];
                } else {
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (n0 + r < N) {
                            if (OPT && out.bf16) reinterpret_cast<uint16_t *>(out.y)[o + r] = bf16_rne(v[r]);
                            else reinterpret_cast<float *>(out.y)[o + r] = v[r];
                            if (acc_out) acc_out[o + r] = acc[i][j][r];
                        }
                    }
                }
            }
        }
    };

    // prologue, matching the producers' barrier: steps 0 and 1 staged
    asm volatile("s_barrier" ::: "memory");
    read(0, 0);
    // iteration s: half 0 of step s is in registers; read half 1 of step s and
    // run half 0, read half 0 of step s + 1 and run half 1.  Past the last step the
    // reads fetch stale (in-range) LDS that is never used: no branch in the loop.
    for (int s = 0; s < total; ++s) {
        read(s, 1);
        half(0);
        if (GRP) fold_half(s, 0);
        read(s + 1, 0);
        half(1);
        if (GRP) fold_half(s, 1);
        if (++c_kk == KS) {
            // products ran on the codes c: acc = sum q c - sum q, the row sums of q
            // formed by the producers while staging this tile (GRP: group by group)
            if (!GRP) {
                #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = sqbuf[c_ti & 3][64 * wm + 16 * i + l16];
                    #pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] -= pv4i{t, t, t, t};
                }
            }
            epilogue(c_ti);
            #pragma unroll
            for (int i = 0; i < 4; ++i)
                #pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j] = pv4i{0, 0, 0, 0};
                    if (GRP) facc[i][j] = pv4f{0.0f, 0.0f, 0.0f, 0.0f};
                }
            c_kk = 0;
            if (++c_ti < my_tiles) load_sx(c_ti);
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
}

// Tile width by a cost model: tiles are dealt to G = min(tiles, CUs) persistent
// workgroups; the busiest one does ceil(tiles / G) tiles.  A k-step of a 128 x 160
// tile takes about 0.78 of one of a 128 x 224 tile (measured over M = 512 .. 4096,
// N = 640 .. 13824, K = 2560 .. 8192 with every CU busy); take the smaller
// busiest-CU time (ties: the wider tile).
static int pipe_pick_tn(int64_t M, int64_t N, int cus, int64_t *tiles_out, int64_t *rounds_out) {
    int best = 7;
    int64_t best_cost = -1;
    for (int tn : {7, 5}) {
        const int64_t bn = 32 * tn;
        const int64_t tiles = ((M + kPipeBM - 1) / kPipeBM) * ((N + bn - 1) / bn);
        const int64_t rounds = (tiles + cus - 1) / cus;
        const int64_t cost = rounds * (tn == 7 ? 100 : 78);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = tn;
            if (tiles_out) *tiles_out = tiles;
            if (rounds_out) *rounds_out = rounds;
        }
    }
    return best;
}

static int device_cus() {
    static int cached[kMaxScratchDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

bool gemm_pipe_ok(int64_t M, int64_t N, int64_t K) {
    // whole 128-weight steps; 32-bit per-lane load offsets within a tile (128 rows of q)
    return K % kPipeKS == 0 && M > 0 && N > 0 && (int64_t)kPipeBM * K < ((int64_t)1 << 31);
}

bool gemm_pipe_groups_ok(int64_t M, int64_t N, int64_t K, int64_t w_group) {
    // group-wise scales: whole groups of half steps (64) or of steps (multiples of 128)
    return gemm_pipe_ok(M, N, K) && w_group > 0 && w_group < K && K % w_group == 0 &&
           (w_group == 64 || w_group % kPipeKS == 0);
}

int64_t gemm_pipe_rounds(int64_t M, int64_t N) {
    int64_t tiles = 0, rounds = 0;
    pipe_pick_tn(M, N, 256, &tiles, &rounds);
    return rounds;
}

double gemm_pipe_estimate_us(int64_t M, int64_t N, int64_t K) {
    int64_t tiles = 0, rounds = 0;
    const int tn = pipe_pick_tn(M, N, 256, &tiles, &rounds);
    // per 128-weight step: about 0.9 us (128 x 224) and 0.7 us (128 x 160) with few
    // workgroups, up to 1.15 and 0.8 us with every CU busy; about 5 us of launch,
    // pipeline fill and epilogue
    const double fill = (double)std::min<int64_t>(tiles, 256) / 256.0;
    const double step = tn == 7 ? 0.9 + 0.25 * fill : 0.7 + 0.1 * fill;
    return (double)rounds * (double)(K / kPipeKS) * step + 5.0;
}

// paired weight loads where the steps of a tile pair up (K a multiple of 256)
static bool pipe_pairs(int64_t K) { return K % (2 * kPipeKS) == 0; }

template <int TN, bool PW>
static void launch_pipe_pw(bool opt, dim3 g, hipStream_t st, const int8_t *q, const float *s_x,
                           const uint8_t *packed, const float *s_w, int m, int n, int k, const OutSpec &y,
                           int32_t *acc, int tiles_m, int nt) {
    if (opt)
        gemm_pipe_kernel<TN, true, false, PW><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, m, n, k, y, acc,
                                                                             tiles_m, nt);
    else
        gemm_pipe_kernel<TN, false, false, PW><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, m, n, k, y, acc,
                                                                              tiles_m, nt);
}

template <int TN>
static void launch_pipe(bool opt, dim3 g, hipStream_t st, const int8_t *q, const float *s_x, const uint8_t *packed,
                        const float *s_w, int m, int n, int k, const OutSpec &y, int32_t *acc, int tiles_m, int nt) {
    if (pipe_pairs(k)) launch_pipe_pw<TN, true>(opt, g, st, q, s_x, packed, s_w, m, n, k, y, acc, tiles_m, nt);
    else launch_pipe_pw<TN, false>(opt, g, st, q, s_x, packed, s_w, m, n, k, y, acc, tiles_m, nt);
}

hipError_t launch_gemm_pipe(int tn_force, const int8_t *q, const float *s_x, const uint8_t *packed,
                            const float *s_w, int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc,
                            hipStream_t st) {
    const int cus = device_cus();
    const bool grp = y.w_group > 0 && y.w_group < K;
    if (grp) {
        // group-wise scales: 128 x 160 tiles (their fp32 group accumulators fit beside
        // the int32 ones), no int32 output
        if (acc || !gemm_pipe_groups_ok(M, N, K, y.w_group)) return hipErrorInvalidValue;
        const int tiles_m = (int)((M + kPipeBM - 1) / kPipeBM);
        const int64_t tiles = (int64_t)tiles_m * ((N + 159) / 160);
        const dim3 g((unsigned)std::min<int64_t>(tiles, cus));
        const bool sgn = BITNET_PIPE_SGN && y.w_group <= 128;
        if (pipe_pairs(K) && sgn)
            gemm_pipe_kernel<5, true, true, true, true><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, (int)M, (int)N,
                                                                                      (int)K, y, nullptr, tiles_m, (int)tiles);
        else if (pipe_pairs(K))
            gemm_pipe_kernel<5, true, true, true><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, (int)M, (int)N,
                                                                                (int)K, y, nullptr, tiles_m, (int)tiles);
        else if (sgn)
            gemm_pipe_kernel<5, true, true, false, true><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, (int)M,
                                                                                       (int)N, (int)K, y, nullptr,
                                                                                       tiles_m, (int)tiles);
        else
            gemm_pipe_kernel<5, true, true, false><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, (int)M, (int)N,
                                                                                 (int)K, y, nullptr, tiles_m, (int)tiles);
        return hipGetLastError();
    }
    const int tn = tn_force ? tn_force : pipe_pick_tn(M, N, cus, nullptr, nullptr);
    const int64_t bn = 32 * tn;
    const int tiles_m = (int)((M + kPipeBM - 1) / kPipeBM);
    const int64_t tiles = (int64_t)tiles_m * ((N + bn - 1) / bn);
    const dim3 g((unsigned)std::min<int64_t>(tiles, cus));
    const bool opt = y.bias || y.bf16 || y.w_group;
    if (tn == 7) launch_pipe<7>(opt, g, st, q, s_x, packed, s_w, (int)M, (int)N, (int)K, y, acc, tiles_m, (int)tiles);
    else launch_pipe<5>(opt, g, st, q, s_x, packed, s_w, (int)M, (int)N, (int)K, y, acc, tiles_m, (int)tiles);
    return hipGetLastError();
}

}  // namespace bitnet
