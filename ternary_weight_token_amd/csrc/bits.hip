// Other encodings of the weights of the same product, each with its own packer and
// contraction:
//  - b1.0 binary weights {-1, +1} (page chenxutan.com sec. 1 and the b1.0 paragraph
//    of sec. 2.1: the first BitNet, no zero), one bit per weight, bit set for +1, LSB first; the scale is the same
//    absmean s_w as for ternary weights;
//  - sign / mask bitplanes (page devpress.csdn.net, sec. "三值量化：把乘法变成加减法":
//    bitnet_linear over weight_sign and weight_mask): per 32 weights a mask word
//    (bit set: nonzero) and a sign word (bit set: -1), converted from the 2-bit
//    codes.
// y = fp32(acc s_x s_w / 127) as for the 2-bit codes (chenxutan.com sec. 2.3).
//
// Contraction (M = 1 GEMV): bit-serial.  The row of q is staged in LDS as its 8
// two's-complement bit planes (plane j of 32 values: bit i = bit j of q_i), and a
// 32-weight word w contributes popcount(plane_j & w) to counter j; at the end
// sum_k q_k [bit k of w] = sum_j 2^j cnt_j with the weight of plane 7 being -128.
// Binary: sum q t = 2 sum_{bit set} q - sum q.  Bitplanes: a negative weight adds
// -q = ~q + 1 (two's complement), so with pos = mask & ~sign each plane word
// becomes bfi(p_j, pos, sign) = (p_j & pos) | (~p_j & sign) -- q's bit where the
// weight is +1, its complement where it is -1, 0 where it is 0 -- and sum q t =
// sum_j 2^j cnt_j + popcount(sign).  Per 32 weights and row that is 16 VALU
// operations (binary) or 19 (bitplanes), no unpacking into bytes.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace bitnet {

// ---- packing

// One thread per 32-weight word: bit i set when w[32 c + i] >= 0 (both zeros give
// +1); words are consecutive over the flat array (K % 32 == 0 keeps them in rows).
__global__ __launch_bounds__(256) void pack_binary_kernel(const float *__restrict__ w, int64_t words,
                                                          uint32_t *__restrict__ bits) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= words) return;
    const float4 *p = reinterpret_cast<const float4 *>(w + 32 * c);
    uint32_t b = 0;
    #pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = p[i];
        b |= (v.x >= 0.0f ? 1u : 0u) << (4 * i);
        b |= (v.y >= 0.0f ? 2u : 0u) << (4 * i);
        b |= (v.z >= 0.0f ? 4u : 0u) << (4 * i);
        b |= (v.w >= 0.0f ? 8u : 0u) << (4 * i);
    }
    bits[c] = b;
}

// One thread per 32 weights (8 bytes of 2-bit codes): code 1 is zero, code 0 is -1,
// codes 2 and 3 are positive (3, never written by the packer, becomes +1).
__global__ __launch_bounds__(256) void pack_bitplanes_kernel(const uint2 *__restrict__ packed, int64_t chunks,
                                                             uint2 *__restrict__ planes) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const uint2 v = packed[c];
    uint32_t mask = 0, sign = 0;
    #pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t code = ((i < 16 ? v.x : v.y) >> (2 * (i & 15))) & 3u;
        mask |= (code != 1u ? 1u : 0u) << i;
        sign |= (code == 0u ? 1u : 0u) << i;
    }
    planes[c] = make_uint2(mask, sign);
}

hipError_t launch_pack_binary(const float *w, int64_t N, int64_t K, uint8_t *bits, hipStream_t st) {
    const int64_t words = N * K / 32;
    if (words == 0) return hipSuccess;
    pack_binary_kernel<<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st>>>(
        w, words, reinterpret_cast<uint32_t *>(bits));
    return hipGetLastError();
}

hipError_t launch_pack_bitplanes(const uint8_t *packed, int64_t N, int64_t K, uint8_t *planes, hipStream_t st) {
    const int64_t chunks = N * K / 32;
    if (chunks == 0) return hipSuccess;
    pack_bitplanes_kernel<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st>>>(
        reinterpret_cast<const uint2 *>(packed), chunks, reinterpret_cast<uint2 *>(planes));
    return hipGetLastError();
}

// ---- bit planes of q

// 8 x 8 bit-matrix transpose of a 64-bit word whose byte r is row r: afterwards
// byte c holds, in bit r, bit c of input byte r.  Three rounds exchange the
// off-diagonal blocks of 1 x 1, 2 x 2 and 4 x 4 bits (masked xor swaps).
__device__ __forceinline__ uint64_t transpose8x8(uint64_t x) {
    uint64_t t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
    x ^= t ^ (t << 7);
    t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
    x ^= t ^ (t << 14);
    t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
    x ^= t ^ (t << 28);
    return x;
}

// The 8 bit planes of 32 int8 values (a, b: bytes 0-15 and 16-31): p[j] bit i =
// bit j of value i.
__device__ __forceinline__ void q_planes(uint4 a, uint4 b, uint32_t (&p)[8]) {
    const uint64_t t0 = transpose8x8((uint64_t)a.y << 32 | a.x);
    const uint64_t t1 = transpose8x8((uint64_t)a.w << 32 | a.z);
    const uint64_t t2 = transpose8x8((uint64_t)b.y << 32 | b.x);
    const uint64_t t3 = transpose8x8((uint64_t)b.w << 32 | b.z);
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int sh = 8 * j;
        p[j] = (uint32_t)((t0 >> sh) & 0xFF) | (uint32_t)((t1 >> sh) & 0xFF) << 8 |
               (uint32_t)((t2 >> sh) & 0xFF) << 16 | (uint32_t)((t3 >> sh) & 0xFF) << 24;
    }
}

// sum_j 2^j cnt_j, plane 7 weighing -128 (two's complement).
__device__ __forceinline__ int plane_sum(const int (&cnt)[8]) {
    int s = -(cnt[7] << 7);
    #pragma unroll
    for (int j = 0; j < 7; ++j) s += cnt[j] << j;
    return s;
}

// ---- M = 1 GEMV

// FMT 1: binary, a 16-byte load is 4 words = 128 weights; FMT 2: bitplanes, a
// 16-byte load is 2 (mask, sign) pairs = 64 weights.  An octet of lanes reads 8
// consecutive 16-byte slots of a row per step; RG rows per octet, 8 octets per
// wave, waves split K into ks slices.  The staged planes of one slot take
// 8 GC + 4 dwords of LDS (the 4 of padding make the 8 slots an octet reads at once
// fall in distinct banks).
template <int FMT>
struct BitsFmt {
    static constexpr int GC = FMT == 1 ? 4 : 2;       // 32-value chunks per 16-byte slot
    static constexpr int SD = 8 * GC + 4;              // LDS dwords per slot
    static constexpr int V = 32 * GC;                  // values per slot
    static constexpr int RowDiv = FMT == 1 ? 8 : 4;    // weights per byte
};

// rows per octet: 4 for tall matrices (fewer LDS plane reads and less loop overhead
// per weight), 2 otherwise (twice the workgroups for a small N)
constexpr int64_t kBitsTallN = 16384;

// Stagers put the bit planes of the token row into LDS (slot layout of BitsFmt):
// load() issues the global loads the staging needs, before the first weight loads
// (so that waiting for them does not wait for the weights); operator() forms the
// planes and, for binary weights, adds the row's sum of q to *sq.

// From int8 q in memory.
template <int FMT>
struct StagePlanesQ {
    const int8_t *q;
    int K;
    struct Pre { uint4 a, b; };
    __device__ __forceinline__ Pre load() const {
        const int c0 = min((int)threadIdx.x, (K >> 5) - 1);
        return Pre{gload16(q + 32 * c0), gload16(q + 32 * c0 + 16)};
    }
    __device__ __forceinline__ void operator()(const Pre &pre, uint32_t *lds, int *sq) const {
        using F = BitsFmt<FMT>;
        const int tid = threadIdx.x, C32 = K >> 5;
        int part = 0;
        auto put = [&](int c, uint4 a, uint4 b) {
            uint32_t p[8];
            q_planes(a, b, p);
            uint32_t *dst = lds + (c / F::GC) * F::SD + 8 * (c % F::GC);
            *reinterpret_cast<uint4 *>(dst) = make_uint4(p[0], p[1], p[2], p[3]);
            *reinterpret_cast<uint4 *>(dst + 4) = make_uint4(p[4], p[5], p[6], p[7]);
            if (FMT == 1) {
                int s = dot4(a.x, 0x01010101u, 0);
                s = dot4(a.y, 0x01010101u, s);
                s = dot4(a.z, 0x01010101u, s);
                s = dot4(a.w, 0x01010101u, s);
                s = dot4(b.x, 0x01010101u, s);
                s = dot4(b.y, 0x01010101u, s);
                s = dot4(b.z, 0x01010101u, s);
                part += dot4(b.w, 0x01010101u, s);
            }
        };
        if (tid < C32) put(tid, pre.a, pre.b);
        for (int c = tid + 256; c < C32; c += 256) put(c, gload16(q + 32 * c), gload16(q + 32 * c + 16));
        if (FMT == 1 && part != 0) atomicAdd(sq, part);
    }
};

// From the bf16 token row (bitplane weights): the absmax quantization of
// bitnet_quant_act done in the workgroup (page chenxutan.com sec. 2.2: s = max|x| as
// an integer max of the bf16 magnitudes, codes rint((127 x) / s), all zero for a zero
// row), then the planes of the codes.  s goes to *s_lds; q and s are also written out
// when q_out / s_out are set.  Each thread holds its first 32 values from load().
template <int FMT>
struct StagePlanesQuant {
    const uint16_t *x;
    int K;
    int8_t *q_out;
    float *s_out;
    float *s_lds;
    uint32_t *red;       // LDS, one word per wavefront
    struct Pre { uint4 v[4]; };
    __device__ __forceinline__ Pre load() const {
        const int c0 = min((int)threadIdx.x, (K >> 5) - 1);   // a clamped duplicate leaves the max as it is
        Pre p;
        #pragma unroll
        for (int i = 0; i < 4; ++i) p.v[i] = gload16(x + 32 * c0 + 8 * i);
        return p;
    }
    __device__ __forceinline__ void operator()(const Pre &pre, uint32_t *lds, int *) const {
        using F = BitsFmt<FMT>;
        static_assert(FMT == 2, "the row sum of q is not formed here");
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, C32 = K >> 5;
        uint32_t mx = max(max(absmax8(pre.v[0]), absmax8(pre.v[1])), max(absmax8(pre.v[2]), absmax8(pre.v[3])));
        for (int c = tid + 256; c < C32; c += 256) {
            #pragma unroll
            for (int i = 0; i < 4; ++i) mx = max(mx, absmax8(gload16(x + 32 * c + 8 * i)));
        }
        mx = wave_max_u32(mx);
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        mx = max(max(red[0], red[1]), max(red[2], red[3]));
        const float s = bf16f(mx);
        const float inv = 1.0f / s;
        if (tid == 0) {
            *s_lds = s;
            if (s_out) *s_out = s;
        }
        auto put = [&](int c, const uint4 (&v)[4]) {
            uint2 w[4] = {make_uint2(0u, 0u), make_uint2(0u, 0u), make_uint2(0u, 0u), make_uint2(0u, 0u)};
            if (mx != 0) {
                #pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = qcode8(v[i], s, inv);
            }
            const uint4 a = make_uint4(w[0].x, w[0].y, w[1].x, w[1].y), b = make_uint4(w[2].x, w[2].y, w[3].x, w[3].y);
            if (q_out) {
                *reinterpret_cast<uint4 *>(q_out + 32 * c) = a;
                *reinterpret_cast<uint4 *>(q_out + 32 * c + 16) = b;
            }
            uint32_t p[8];
            q_planes(a, b, p);
            uint32_t *dst = lds + (c / F::GC) * F::SD + 8 * (c % F::GC);
            *reinterpret_cast<uint4 *>(dst) = make_uint4(p[0], p[1], p[2], p[3]);
            *reinterpret_cast<uint4 *>(dst + 4) = make_uint4(p[4], p[5], p[6], p[7]);
        };
        if (tid < C32) put(tid, pre.v);
        for (int c = tid + 256; c < C32; c += 256) {
            const uint4 v[4] = {gload16(x + 32 * c), gload16(x + 32 * c + 8), gload16(x + 32 * c + 16),
                                gload16(x + 32 * c + 24)};
            put(c, v);
        }
    }
};

// One token row against rows [row_base, row_base + (4 / ks) 8 RG) of the weights.
// sxp is read after the staging (it may be the LDS word the stager writes).
template <int FMT, int RG, class Stage>
__device__ __forceinline__ void bits_tile(const Stage &stage, const float *sxp, const uint8_t *__restrict__ wbits,
                                          const float *__restrict__ s_w, int N, int K, int row_base, int ks,
                                          float *__restrict__ y, int32_t *__restrict__ acc_out, uint32_t *lds,
                                          int *sq_ptr, int *red) {
    using F = BitsFmt<FMT>;
    int &sq = *sq_ptr;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l8 = lane & 7, rs = lane >> 3;
    const int S = K / F::V;
    const int rowsets = 4 / ks, rowset = wave / ks, slice = wave - rowset * ks;
    const int row0 = row_base + rowset * 8 * RG;
    const int sb = (int)((int64_t)S * slice / ks), se = (int)((int64_t)S * (slice + 1) / ks);
    const int64_t row_bytes = K / F::RowDiv;

    const uint8_t *prow[RG];
    #pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int r = row0 + 8 * g + rs;
        prow[g] = wbits + (size_t)(r < N ? r : 0) * row_bytes;   // rows past N read row 0, discarded
    }
    const int T = row0 < N && se > sb ? (se - sb + 7) >> 3 : 0;
    const int slast = max(se - 1, 0);
    uint4 bufA[RG], bufB[RG];
    auto issue = [&](uint4 (&b)[RG], int t) {
        const int sl = min(sb + l8 + 8 * t, slast);
        #pragma unroll
        for (int g = 0; g < RG; ++g) b[g] = load_weights<true>(prow[g] + 16 * (size_t)sl);
    };

    // the stager's loads, then the first weights, then the staging
    const typename Stage::Pre pre = stage.load();
    issue(bufA, 0);
    if (tid == 0) sq = 0;
    __syncthreads();   // sq initialised
    stage(pre, lds, &sq);
    __syncthreads();

    // counters per row and plane (bitplanes: and of the sign bits)
    int cnt[RG][8], cns[RG];
    #pragma unroll
    for (int g = 0; g < RG; ++g) {
        cns[g] = 0;
        #pragma unroll
        for (int j = 0; j < 8; ++j) cnt[g][j] = 0;
    }
    // CHECK: the step may hold slots past the slice (only the last one does); they
    // count as all-zero words
    auto consume = [&](const uint4 (&b)[RG], int t, auto check) {
        constexpr bool CHECK = decltype(check)::value;
        const int sl = sb + l8 + 8 * t;
        const bool valid = !CHECK || sl < se;
        const uint32_t *src = lds + (CHECK ? min(sl, slast) : sl) * F::SD;
        #pragma unroll
        for (int i = 0; i < F::GC; ++i) {
            const uint4 p0 = *reinterpret_cast<const uint4 *>(src + 8 * i);
            const uint4 p1 = *reinterpret_cast<const uint4 *>(src + 8 * i + 4);
            const uint32_t p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            #pragma unroll
            for (int g = 0; g < RG; ++g) {
                const uint32_t wv[4] = {b[g].x, b[g].y, b[g].z, b[g].w};
                if (FMT == 1) {
                    const uint32_t w = valid ? wv[i] : 0u;
                    #pragma unroll
                    for (int j = 0; j < 8; ++j) cnt[g][j] += __builtin_popcount(p[j] & w);
                } else {
                    const uint32_t m = valid ? wv[2 * i] : 0u;
                    const uint32_t sg = m & wv[2 * i + 1];   // a sign bit counts only under the mask
                    const uint32_t pos = m ^ sg;
                    #pragma unroll
                    for (int j = 0; j < 8; ++j) cnt[g][j] += __builtin_popcount((p[j] & pos) | (~p[j] & sg));
                    cns[g] += __builtin_popcount(sg);
                }
            }
        }
    };
    using Checked = std::true_type;
    using Unchecked = std::false_type;
    // two register buffers: the loads of step t + 1 are in flight during step t;
    // every slot of steps 0 .. T - 2 lies inside the slice
    if (T > 0) {
        int t = 0;
        for (; t + 2 <= T - 1; t += 2) {
            issue(bufB, t + 1);
            consume(bufA, t, Unchecked{});
            issue(bufA, t + 2);
            consume(bufB, t + 1, Unchecked{});
        }
        if (t == T - 2) {
            issue(bufB, t + 1);
            consume(bufA, t, Unchecked{});
            consume(bufB, t + 1, Checked{});
        } else {
            consume(bufA, t, Checked{});
        }
    }

    int a[RG];
    #pragma unroll
    for (int g = 0; g < RG; ++g) a[g] = octet_sum(plane_sum(cnt[g]) + cns[g]);
    const double c = rescale_factor(*sxp, *s_w);
    auto finish = [&](int r, int v) {
        const int acc = FMT == 1 ? 2 * v - sq : v;
        y[r] = rescale(acc, c);
        if (acc_out) acc_out[r] = acc;
    };
    if (ks == 1) {
        #pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int r = row0 + 8 * g + rs;
            if (l8 == 0 && r < N) finish(r, a[g]);
        }
        return;
    }
    constexpr int R = 8 * RG;
    if (l8 == 0) {
        #pragma unroll
        for (int g = 0; g < RG; ++g) red[wave * R + 8 * g + rs] = a[g];
    }
    __syncthreads();
    if (tid < rowsets * R) {
        const int rsi = tid / R, rr = tid - rsi * R;
        const int r = row_base + rsi * R + rr;
        if (r < N) {
            int v = 0;
            for (int w = 0; w < ks; ++w) v += red[(rsi * ks + w) * R + rr];
            finish(r, v);
        }
    }
}

// Binary with 4 rows per octet is held at 4 waves per SIMD (it would settle just
// above 128 registers otherwise); the bitplane kernels run faster as compiled.
template <int FMT, int RG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FMT == 1 && RG == 4 ? 4 : 1)))
void gemv_bits_kernel(const int8_t *__restrict__ q, const float *__restrict__ s_x, const uint8_t *__restrict__ wbits,
                      const float *__restrict__ s_w, int N, int K, float *__restrict__ y,
                      int32_t *__restrict__ acc_out, int ks) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    __shared__ int sq;
    __shared__ int red[4 * 8 * RG];
    bits_tile<FMT, RG>(StagePlanesQ<FMT>{q, K}, s_x, wbits, s_w, N, K, (int)blockIdx.x * ((4 / ks) * 8 * RG), ks, y,
                       acc_out, lds, &sq, red);
}

// Fused decode step over bitplane weights: the block table and descriptors of the
// fused grouped plan (one token row per problem, 4 rows per octet, no K split), the
// row quantized in every workgroup of its problem while staging its planes.
constexpr int kBitsFusedRG = 4;

__global__ __launch_bounds__(256) void gemv_bits_fused_grouped_kernel(const uint8_t *__restrict__ plan) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    __shared__ int sq;
    __shared__ int red[4 * 8 * kBitsFusedRG];
    __shared__ uint32_t qred[4];
    __shared__ float s_lds;
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[blockIdx.x];
    const FusedDescDev d = reinterpret_cast<const FusedDescDev *>(plan + h->desc_offset)[e.desc];
    const bool first = e.local == 0;
    bits_tile<2, kBitsFusedRG>(
        StagePlanesQuant<2>{d.x, d.K, first ? d.q : nullptr, first ? d.s_x : nullptr, &s_lds, qred}, &s_lds,
        d.packed, d.s_w, d.N, d.K, (int)e.local * (4 * 8 * kBitsFusedRG), 1, d.y, d.acc, lds, &sq, red);
}

uint32_t bits_fused_rows_per_block() { return 4 * 8 * kBitsFusedRG; }
uint32_t bits_fused_lds_bytes(int64_t K) { return (uint32_t)((K / BitsFmt<2>::V) * BitsFmt<2>::SD * 4); }

hipError_t launch_bits_fused_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, hipStream_t st) {
    gemv_bits_fused_grouped_kernel<<<dim3(blocks), dim3(256), lds_bytes, st>>>(
        reinterpret_cast<const uint8_t *>(plan_dev));
    return hipGetLastError();
}

// Longest K whose staged planes fit 63 KiB of LDS (the kernel's own arrays beside them).
int64_t bits_max_k(int fmt) {
    constexpr int kBytes = 63 * 1024;
    return fmt == 1 ? (int64_t)(kBytes / (BitsFmt<1>::SD * 4)) * BitsFmt<1>::V
                    : (int64_t)(kBytes / (BitsFmt<2>::SD * 4)) * BitsFmt<2>::V;
}

bool bits_fast_ok(int fmt, int64_t M, int64_t K, const void *q, const void *wbits) {
    const int64_t v = fmt == 1 ? BitsFmt<1>::V : BitsFmt<2>::V;
    return M == 1 && K > 0 && K % v == 0 && K <= bits_max_k(fmt) && (uintptr_t)q % 16 == 0 &&
           (uintptr_t)wbits % 16 == 0;
}

template <int FMT, int RG>
static hipError_t launch_gemv_bits_rg(const int8_t *q, const float *s_x, const uint8_t *wbits, const float *s_w,
                                      int64_t N, int64_t K, float *y, int32_t *acc, hipStream_t st) {
    using F = BitsFmt<FMT>;
    const int S = (int)(K / F::V);
    auto blocks = [&](int k) { return (N + (4 / k) * 8 * RG - 1) / ((4 / k) * 8 * RG); };
    // more K slices while the launch has fewer than 2 workgroups per CU and each
    // slice would keep at least 1024 weights of its rows
    int ks = 1;
    while (ks < 4 && blocks(ks) < 512 && K / (2 * ks) >= 1024) ks *= 2;
    const size_t lds = (size_t)S * F::SD * 4;
    gemv_bits_kernel<FMT, RG><<<dim3((unsigned)blocks(ks)), dim3(256), lds, st>>>(q, s_x, wbits, s_w, (int)N, (int)K,
                                                                                  y, acc, ks);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_gemv_bits(const int8_t *q, const float *s_x, const uint8_t *wbits, const float *s_w,
                                   int64_t N, int64_t K, float *y, int32_t *acc, hipStream_t st) {
    return N >= kBitsTallN ? launch_gemv_bits_rg<FMT, 4>(q, s_x, wbits, s_w, N, K, y, acc, st)
                           : launch_gemv_bits_rg<FMT, 2>(q, s_x, wbits, s_w, N, K, y, acc, st);
}

// ---- any M: one thread per output, plain loops (any alignment)

template <int FMT>
__global__ __launch_bounds__(256) void linear_bits_generic_kernel(const int8_t *__restrict__ q,
                                                                  const float *__restrict__ s_x,
                                                                  const uint8_t *__restrict__ wbits,
                                                                  const float *__restrict__ s_w, int64_t M,
                                                                  int64_t N, int64_t K, float *__restrict__ y,
                                                                  int32_t *__restrict__ acc_out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx % N;
    const int8_t *qr = q + m * K;
    int a = 0;
    if (FMT == 1) {
        const uint8_t *br = wbits + n * (K / 8);
        for (int64_t k = 0; k < K; ++k) a += ((br[k >> 3] >> (k & 7)) & 1u) ? qr[k] : -qr[k];
    } else {
        const uint8_t *pr = wbits + n * (K / 4);
        for (int64_t c = 0; c < K / 32; ++c) {
            const uint8_t *ch = pr + 8 * c;
            const uint32_t mask = ch[0] | ch[1] << 8 | ch[2] << 16 | (uint32_t)ch[3] << 24;
            const uint32_t sign = ch[4] | ch[5] << 8 | ch[6] << 16 | (uint32_t)ch[7] << 24;
            for (int i = 0; i < 32; ++i)
                if ((mask >> i) & 1u) a += ((sign >> i) & 1u) ? -qr[32 * c + i] : qr[32 * c + i];
        }
    }
    y[idx] = rescale(a, rescale_factor(s_x[m], *s_w));
    if (acc_out) acc_out[idx] = a;
}

hipError_t launch_linear_bits(const int8_t *q, const float *s_x, const uint8_t *wbits, int fmt, const float *s_w,
                              int64_t M, int64_t N, int64_t K, float *y, int32_t *acc, int kernel, hipStream_t st) {
    const bool fast = kernel == 2 || (kernel == 0 && bits_fast_ok(fmt, M, K, q, wbits));
    if (fast) {
        return fmt == 1 ? launch_gemv_bits<1>(q, s_x, wbits, s_w, N, K, y, acc, st)
                        : launch_gemv_bits<2>(q, s_x, wbits, s_w, N, K, y, acc, st);
    }
    const int64_t total = M * N;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (fmt == 1)
        linear_bits_generic_kernel<1><<<grid, dim3(256), 0, st>>>(q, s_x, wbits, s_w, M, N, K, y, acc);
    else
        linear_bits_generic_kernel<2><<<grid, dim3(256), 0, st>>>(q, s_x, wbits, s_w, M, N, K, y, acc);
    return hipGetLastError();
}

}  // namespace bitnet
