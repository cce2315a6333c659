// Prefill GEMM, pipelined and persistent: the contraction and rescale of the
// BitLinear forward (pages: chenxutan.com sec. 2.3 rescale, sec. 3.1
// BitLinear.forward over the quantized operands) as int8 x ternary -> int32 on
// the matrix cores (v_mfma_i32_16x16x64_i8), for many tokens.
//
// Workgroup: 8 wavefronts, two per SIMD, with two roles; output tile 128 x BN,
// BN = 32 TN weight rows.
//  * 4 consumer waves (2 x 2): each owns 64 token rows x 16 TN weight rows, reads
//    its MFMA operands from LDS and runs the products; at the end of a tile it
//    rescales and stores its block straight from the accumulators (y = fp32(acc
//    c_m), c_m = (s_x s_w) / 127 in float64).
//  * 4 producer waves: move the operands into LDS with direct-to-LDS loads
//    (global_load_lds_dwordx4: no registers in flight) D - 1 k-steps ahead, and
//    expand the packed ternary codes to int8 weights t = c - 1 in LDS one half
//    step to one and a half steps ahead of their use.
// Consumers never issue loads the producers wait for, and producers never
// store, so each role's memory counter holds only its own traffic: the output
// stores of one tile drain while the next tile computes.
//
// One k-step is 128 weights: every row of q and of the packed weights is read in
// whole 128-byte lines (half lines load at half the rate).  A stage holds q for
// 128 rows (16 loads of 8 rows x 128 bytes, lane-linear in LDS, the 16-byte
// chunks of each row XOR-swizzled so that the fragment reads are free of bank
// conflicts) and the packed weights of up to 256 rows (32 bytes each).  Expanded
// weights go to four half-step buffers of 1 KB blocks laid out as the MFMA reads
// them (lane L: row L % 16, bytes 16 (L / 16) .. +15 of the 64-weight half).  The
// MFMA takes the weights as its first operand and the tokens as its second, so
// each lane ends with 4 consecutive output columns of one token row: one 16-byte
// store.
//
// The grid is one workgroup per compute unit; workgroup b takes tiles b, b + G,
// ... in column-major order of M tiles.  The step sequence runs across tile
// boundaries: loads for the next tile start while the current one computes.  The
// k order is rotated per workgroup (the sum over k is order-free), so that
// workgroups reading the same rows are at different k at any moment.
#include "device_common.h"
#include "internal.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace bitnet {

namespace {

typedef int pv4i __attribute__((ext_vector_type(4)));
typedef float pv4f __attribute__((ext_vector_type(4)));

constexpr int kPipeBM = 128;                    // token rows per tile (2 consumer waves x 64)
constexpr int kPipeKS = 128;                    // weights per k-step (one 128-byte line of q per row)
constexpr int kPipeA = kPipeBM * kPipeKS;       // q bytes per stage (16 loads of 1 KB)
constexpr int kPipeBp = 256 * 32;               // packed weight bytes per stage (8 loads of 32 rows)
constexpr int kPipeStage = kPipeA + kPipeBp;
constexpr int kPipeThreads = 512;
constexpr int kPipeLoads = 6;                   // loads per producer wave and step

__device__ __forceinline__ uint32_t lds_offset(const void *p) { return (uint32_t)(uintptr_t)p; }

// 16 bytes per lane from base + voff into LDS at m0 + 16 * lane (lanes of the
// exec mask only).  The load has no destination registers: its completion is
// tracked by the vector memory counter alone.
__device__ __forceinline__ void dma16(uint32_t lds, const void *base, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "m0");
}

// The 4 codes of one packed byte (k = 4j + i in bits 2i..2i+1) spread to 4 bytes in
// k order, byte i = code i: the products run on the codes c and the kernel
// subtracts sum_k q afterwards, sum q (c - 1) = sum q c - sum q (code 3 reads +2).
__device__ __forceinline__ uint32_t spread4(uint32_t byte) {
    const uint32_t sp = byte | (byte << 6);
    return (sp | (sp << 12)) & 0x03030303u;
}

// LDS slot of 16-byte chunk c (0..7) of local q row r within its 128-byte row:
// the chunk index XORed with the row's position, so that the 16 lanes of a
// fragment read (16 rows, one chunk) hit distinct banks.
__device__ __forceinline__ int qslot(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

}  // namespace

// TN: 16-row weight blocks per consumer wave (tile BN = 32 TN); D: stages.
// OPT: the epilogue options (bias, bf16 output, one weight scale per output
// channel) are compiled in; without them the store path is fp32 y (and acc).
template <int TN, int D, bool OPT>
__global__ __launch_bounds__(kPipeThreads, 1) void gemm_pipe_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s_x, const uint8_t *__restrict__ packed,
    const float *__restrict__ s_w, int M, int N, int K, const OutSpec out, int32_t *__restrict__ acc_out,
    int tiles_m, int n_tiles) {
    constexpr int BN = 32 * TN;
    static_assert(BN <= 256, "packed stage holds 256 rows");
    static_assert(D >= 4, "the wait before each barrier covers the step three ahead");
    constexpr int HB = BN * 64;                  // expanded weights of one half step
    __shared__ __attribute__((aligned(1024))) uint8_t smem[D * kPipeStage + 4 * HB];
    uint8_t *const expb = smem + D * kPipeStage;

    // the wave index is the same in every lane: keep it (and what derives from it) scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, wg = blockIdx.x;
    const int my_tiles = (n_tiles - wg + G - 1) / G;
    const int KS = K / kPipeKS;
    const int total = my_tiles * KS;
    const size_t KB = (size_t)(K >> 2);

    if (wave >= 4) {
        // ------------------------------------------------------------ producer
        const int p = wave - 4;
        const int tp = tid - 256;
        int d_s = 0, d_ti = 0, d_kk = 0;
        // k order rotated per workgroup: workgroups that share q rows (one XCD,
        // one M tile) or weight rows (one N tile) start at different k
        const int kx = wg & 7, kj = wg >> 3, kjn = (G + 7) >> 3;
        int d_kr = (int)(((int64_t)kj * KS / kjn + 3 * kx) % KS);
        const int8_t *a_base = nullptr;
        const uint8_t *b_base = nullptr;
        uint32_t a_off[4], b_off[2];
        auto set_tile = [&](int ti) {
            const int t = wg + ti * G;
            const int m0 = (t % tiles_m) * kPipeBM, n0 = (t / tiles_m) * BN;
            a_base = q + (size_t)m0 * K;
            b_base = packed + (size_t)n0 * KB;
            #pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int i = 4 * p + b;                              // load i: local rows 8i .. 8i + 7
                const int r = 8 * i + (lane >> 3);
                const int c = qslot(r, lane & 7);                     // slot lane % 8 holds chunk c
                a_off[b] = (uint32_t)(min(m0 + r, M - 1) - m0) * (uint32_t)K + 16u * (uint32_t)c;
            }
            #pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int r = 32 * (p + 4 * b) + (lane >> 1);         // load p + 4b: local rows 32 (p + 4b) ..
                b_off[b] = (uint32_t)(min(n0 + r, N - 1) - n0) * (uint32_t)KB + 16u * (uint32_t)(lane & 1);
            }
        };
        set_tile(0);
        // the loads of step d_s (clamped to the last step) into its stage
        auto issue = [&]() {
            const uint32_t st = lds_offset(smem) + (uint32_t)((d_s % D) * kPipeStage);
            const int8_t *ab = a_base + (size_t)d_kr * kPipeKS;
            const uint8_t *bb = b_base + (size_t)d_kr * (kPipeKS / 4);
            #pragma unroll
            for (int b = 0; b < 4; ++b) dma16(st + (uint32_t)((4 * p + b) * 1024), ab, a_off[b]);
            #pragma unroll
            for (int b = 0; b < 2; ++b) dma16(st + (uint32_t)(kPipeA + (p + 4 * b) * 1024), bb, b_off[b]);
            ++d_s;
            if (d_s < total) {
                if (++d_kr == KS) d_kr = 0;
                if (++d_kk == KS) {
                    d_kk = 0;
                    set_tile(++d_ti);
                }
            }
        };
        // Expansion task tau of a half step: 16 weights (one packed dword) of weight
        // row r, chunk c of the half; its 16 bytes go to 16 tau of the half buffer
        // (block tau / 64 = 16-row block, lane-linear inside).  bp: the stage's packed
        // rows at this half's 16 bytes.
        auto task_src = [&](const uint8_t *bp, int tau) {
            const int r = 16 * (tau >> 6) + (tau & 15), c = (tau >> 4) & 3;
            return bp + 1024 * (r >> 5) + 32 * (r & 31) + 4 * c;
        };
        auto tern16 = [&](uint32_t w) {
            return make_uint4(spread4(w & 0xFFu), spread4((w >> 8) & 0xFFu), spread4((w >> 16) & 0xFFu), spread4(w >> 24));
        };
        // expand half u of step x into half buffer (2x + u) % 4 (prologue only)
        auto expand = [&](int x, int u) {
            const uint8_t *bp = smem + (x % D) * kPipeStage + kPipeA + 16 * u;
            uint8_t *eb = expb + ((2 * x + u) & 3) * HB;
            #pragma unroll
            for (int h = 0; h < (4 * BN + 255) / 256; ++h) {
                const int tau = tp + 256 * h;
                if (tau < 4 * BN)
                    *reinterpret_cast<uint4 *>(eb + 16 * tau) = tern16(*reinterpret_cast<const uint32_t *>(task_src(bp, tau)));
            }
        };
        // The loop's two half steps, half 1 of step x and half 0 of step x + 1, as one
        // set of 8 BN / 256 tasks per thread (7 or 5: no remainder), all LDS reads
        // first, then the arithmetic, then the stores: no branches, the read latency
        // paid once.
        constexpr int NT2 = 8 * BN / 256;
        static_assert(8 * BN % 256 == 0, "two half steps split evenly over the producers");
        auto expand_pair = [&](int x) {
            const uint8_t *bp1 = smem + (x % D) * kPipeStage + kPipeA + 16;
            const uint8_t *bp0 = smem + ((x + 1) % D) * kPipeStage + kPipeA;
            uint8_t *eb1 = expb + ((2 * x + 1) & 3) * HB, *eb0 = expb + ((2 * x + 2) & 3) * HB;
            uint32_t w[NT2];
            #pragma unroll
            for (int h = 0; h < NT2; ++h) {
                const int tau = tp + 256 * h;
                w[h] = *reinterpret_cast<const uint32_t *>(tau < 4 * BN ? task_src(bp1, tau) : task_src(bp0, tau - 4 * BN));
            }
            // the same operation across all tasks, one stage at a time: independent
            // instructions back to back instead of one dependent chain per byte
            uint32_t e[NT2][4];
            #pragma unroll
            for (int h = 0; h < NT2; ++h) {
                e[h][0] = w[h] & 0xFFu;
                e[h][1] = (w[h] >> 8) & 0xFFu;
                e[h][2] = (w[h] >> 16) & 0xFFu;
                e[h][3] = w[h] >> 24;
            }
            #pragma unroll
            for (int h = 0; h < NT2; ++h)
                #pragma unroll
                for (int d = 0; d < 4; ++d) e[h][d] |= e[h][d] << 6;
            #pragma unroll
            for (int h = 0; h < NT2; ++h)
                #pragma unroll
                for (int d = 0; d < 4; ++d) e[h][d] = (e[h][d] | (e[h][d] << 12)) & 0x03030303u;
            #pragma unroll
            for (int h = 0; h < NT2; ++h) {
                const int tau = tp + 256 * h;
                uint8_t *dst = tau < 4 * BN ? eb1 + 16 * tau : eb0 + 16 * (tau - 4 * BN);
                *reinterpret_cast<uint4 *>(dst) = make_uint4(e[h][0], e[h][1], e[h][2], e[h][3]);
            }
        };
        for (int i = 0; i < D - 1; ++i) issue();
        // steps 0..2 resident
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPipeLoads * (D - 4)) : "memory");
        expand(0, 0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        expand(0, 1);   // while the consumers read half 0 of step 0
        expand(1, 0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int s = 0; s < total; ++s) {
            // step s + D - 1 into the stage of step s - 1 (read up to the last barrier);
            // half 1 of step s + 1 and half 0 of step s + 2 into the buffers of step
            // s - 1's half 1 and step s's half 0 (read up to the last barrier)
            issue();
            expand_pair(s + 1);
            // step s + 3 resident: the next iteration expands from it
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPipeLoads * (D - 4)) : "memory");
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
    // per-lane offset of the q fragment of half u: local row r = 64 wm + 16 i + l16
    // lies in load r / 8 at position r % 8 = lane % 8, chunk 4u + g at its slot
    int aoff[2];
    #pragma unroll
    for (int u = 0; u < 2; ++u)
        aoff[u] = 1024 * ((lane >> 3) & 1) + 128 * (lane & 7) + 16 * qslot(lane & 15, 4 * u + g);
    pv4i fa[2][4], fb[TN];
    // sum of this lane's q bytes per 16-row block i (the lane's k chunks); the four
    // lane groups together cover every k of the tile
    int sq[4] = {0, 0, 0, 0};
    auto sum_q = [&](int set) {
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            int t = __builtin_amdgcn_sdot4(fa[set][i].x, 0x01010101, sq[i], false);
            t = __builtin_amdgcn_sdot4(fa[set][i].y, 0x01010101, t, false);
            t = __builtin_amdgcn_sdot4(fa[set][i].z, 0x01010101, t, false);
            sq[i] = __builtin_amdgcn_sdot4(fa[set][i].w, 0x01010101, t, false);
        }
    };
    auto read_a = [&](int x, int u, int set) {
        const uint8_t *st = smem + (x % D) * kPipeStage + 1024 * (8 * wm) + aoff[u];
        #pragma unroll
        for (int i = 0; i < 4; ++i) fa[set][i] = *reinterpret_cast<const pv4i *>(st + 2048 * i);
    };
    auto read_b = [&](int x, int u, int j) {
        fb[j] = *reinterpret_cast<const pv4i *>(expb + ((2 * x + u) & 3) * HB + 1024 * (TN * wn + j) + 16 * lane);
    };

    const float sw = *s_w;
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
                    double yv = (double)acc[i][j][r] * ((OPT && out.w_group) ? rescale_factor(sxr[i], s_w[n]) : cm);
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

    // prologue, matching the producers' three barriers: steps 0..2 loaded; half 0
    // of step 0 expanded (read here while half 1 of step 0 and half 0 of step 1 are
    // expanded into other buffers); those expanded.
    asm volatile("s_barrier" ::: "memory");
    read_a(0, 0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    #pragma unroll
    for (int j = 0; j < TN; ++j) read_b(0, 0, j);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // iteration s: half 0 of step s is in registers; read and run half 1, reading
    // half 0 of step s + 1 behind it (each weight fragment as soon as its last
    // product has issued)
    // past the last step the reads of step s + 1 fetch stale (in-range) LDS and
    // are never used: no branch in the loop
    for (int s = 0; s < total; ++s) {
        read_a(s, 1, 1);
        sum_q(0);
        #pragma unroll
        for (int j = 0; j < TN; ++j) {
            #pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[j], fa[0][i], acc[i][j], 0, 0, 0);
            read_b(s, 1, j);
        }
        sum_q(1);
        read_a(s + 1, 0, 0);
        #pragma unroll
        for (int j = 0; j < TN; ++j) {
            #pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[j], fa[1][i], acc[i][j], 0, 0, 0);
            read_b(s + 1, 0, j);
        }
        if (++c_kk == KS) {
            // products ran on the codes c: acc = sum q c - sum q, the row's sum of q
            // gathered from the four lane groups of each token row
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                int t = sq[i] + __shfl_xor(sq[i], 16, 64);
                t += __shfl_xor(t, 32, 64);
                #pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] -= pv4i{t, t, t, t};
                sq[i] = 0;
            }
            epilogue(c_ti);
            #pragma unroll
            for (int i = 0; i < 4; ++i)
                #pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = pv4i{0, 0, 0, 0};
            c_kk = 0;
            if (++c_ti < my_tiles) load_sx(c_ti);
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
}

// Tile width by a cost model: tiles are dealt to G = min(tiles, CUs) persistent
// workgroups; the busiest one does ceil(tiles / G) tiles of 128 x BN outputs.
// Among BN = 224 and 160, take the smaller busiest-CU work (ties: the wider tile).
static int pipe_pick_tn(int64_t M, int64_t N, int cus, int64_t *tiles_out, int64_t *rounds_out) {
    int best = 7;
    int64_t best_cost = -1;
    for (int tn : {7, 5}) {
        const int64_t bn = 32 * tn;
        const int64_t tiles = ((M + kPipeBM - 1) / kPipeBM) * ((N + bn - 1) / bn);
        const int64_t rounds = (tiles + cus - 1) / cus;
        const int64_t cost = rounds * bn;
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

double gemm_pipe_estimate_us(int64_t M, int64_t N, int64_t K) {
    int64_t tiles = 0, rounds = 0;
    const int tn = pipe_pick_tn(M, N, 256, &tiles, &rounds);
    // about 0.5 us per 128-weight step of a 128 x 224 tile, 0.4 us of a 128 x 160 tile
    return (double)rounds * (double)(K / kPipeKS) * (tn == 7 ? 0.5 : 0.4) + 5.0;
}

// stages: 4 for the 128 x 224 tile (152 KB of LDS), 5 for 128 x 160 (160 KB)
template <int TN, int D>
static void launch_pipe(bool opt, dim3 g, hipStream_t st, const int8_t *q, const float *s_x, const uint8_t *packed,
                        const float *s_w, int m, int n, int k, const OutSpec &y, int32_t *acc, int tiles_m, int nt) {
    if (opt) gemm_pipe_kernel<TN, D, true><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, m, n, k, y, acc, tiles_m, nt);
    else gemm_pipe_kernel<TN, D, false><<<g, dim3(kPipeThreads), 0, st>>>(q, s_x, packed, s_w, m, n, k, y, acc, tiles_m, nt);
}

hipError_t launch_gemm_pipe(int tn_force, const int8_t *q, const float *s_x, const uint8_t *packed,
                            const float *s_w, int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc,
                            hipStream_t st) {
    const int cus = device_cus();
    const int tn = tn_force ? tn_force : pipe_pick_tn(M, N, cus, nullptr, nullptr);
    const int64_t bn = 32 * tn;
    const int tiles_m = (int)((M + kPipeBM - 1) / kPipeBM);
    const int64_t tiles = (int64_t)tiles_m * ((N + bn - 1) / bn);
    const dim3 g((unsigned)std::min<int64_t>(tiles, cus));
    const bool opt = y.bias || y.bf16 || y.w_group;
    if (tn == 7) launch_pipe<7, 4>(opt, g, st, q, s_x, packed, s_w, (int)M, (int)N, (int)K, y, acc, tiles_m, (int)tiles);
    else launch_pipe<5, 5>(opt, g, st, q, s_x, packed, s_w, (int)M, (int)N, (int)K, y, acc, tiles_m, (int)tiles);
    return hipGetLastError();
}

}  // namespace bitnet
