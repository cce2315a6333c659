// Decode GEMV (M <= 16): acc[m][n] = sum_k q[m][k] * t[n][k], y = acc * s_x * s_w / 127
// (pages: chenxutan.com sec. 2.3 rescale and sec. 3.1 BitLinear.forward; the
// ternary product is an add / subtract / skip, chenxutan.com sec. 1).
//
// HBM-bound: every packed weight byte is read exactly once.  Layout of the work:
//  * a wavefront owns RG row groups of 8 rows; the 8 lanes of an octet walk one
//    row, lane l8 taking 16-byte chunks l8, l8 + 8, ... (one chunk = 64 weights),
//    so one load instruction reads 8 rows x 128 contiguous bytes;
//  * the 2-bit codes c = t + 1 are used unshifted: sum_k q t = sum_k q c - sum_k q,
//    the second term costing a few dot products per chunk and row of q instead of
//    one subtraction per weight;
//  * DOT8 = false: codes regrouped by shift + mask into bytes (codes_i) and fed to
//    v_dot4_i32_i8 against byte-transposed q (7 + 4 VALU ops per 16 weights);
//    DOT8 = true: codes kept as nibbles (2 masks, 1 shift) and fed to the 4-bit
//    dot products against q split into its signed high and unsigned low nibbles
//    (3 + 4 ops per 16 weights);
//  * the 64 q bytes of a chunk are loaded once per chunk (L1/L2-resident),
//    rearranged once and reused by every row group of the wavefront;
//  * partial sums are reduced across the octet with DPP; when the workgroup has
//    several wavefronts they split K and combine their partials through LDS;
//  * epilogue: y = fp32(acc * c_m), c_m = (s_x[m] * s_w) / 127 in float64.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

#ifndef BITNET_GROUPED_RG
#define BITNET_GROUPED_RG 2      // row groups of 8 per wavefront, grouped launch (q staged)
#endif
#ifndef BITNET_FUSED_RG
#define BITNET_FUSED_RG 4        // row groups of 8 per wavefront, fused launch
#endif
#ifndef BITNET_GROUPED_DOT8
#define BITNET_GROUPED_DOT8 1
#endif
#ifndef BITNET_GEMV_NT
#define BITNET_GEMV_NT 1
#endif
#ifndef BITNET_GEMV1_RG
#define BITNET_GEMV1_RG 2        // row groups of 8 per wavefront, single-token launches
#endif
#ifndef BITNET_FUSED_NW
#define BITNET_FUSED_NW 4        // wavefronts per workgroup of the fused grouped launch (4 or 8)
#endif
#ifndef BITNET_FUSED_PERSIST
#define BITNET_FUSED_PERSIST 0   // > 0: the fused grouped launch uses at most this many workgroups
#endif
#ifndef BITNET_GEMV_WG_STORE
#define BITNET_GEMV_WG_STORE 1     // one token: wavefront 0 stores the outputs of the whole workgroup
#endif
#ifndef BITNET_GEMV_PREISSUE
#define BITNET_GEMV_PREISSUE 1   // weight steps issued before the q staging (1 or 2), GEMV launches
#endif
#ifndef BITNET_FUSED_PREISSUE
#define BITNET_FUSED_PREISSUE 2  // the same for the fused grouped launch
#endif

namespace bitnet {

// ---------------------------------------------------------------------------
// LDS-staged variant (used whenever MT x K fits the LDS budget).  A workgroup of
// 4 wavefronts shares one M tile of q: the prologue loads it once, rearranges each
// 16-byte piece (nibble form for the 4-bit dot products, byte transpose for
// v_dot4), stores it in LDS (80 bytes per 64-weight chunk, which keeps the 8
// chunks an instruction reads on distinct banks) and forms sum_k q per row of q.
// The main loop then issues only weight loads to memory, prefetching the next
// chunk's weights before working on the current one.
constexpr int kLdsChunkDw = 20;           // dwords per staged chunk (64 bytes + pad)
constexpr int kLdsBudget = 64 * 1024;     // bytes of staged q per workgroup

template <bool DOT8>
__device__ __forceinline__ uint4 prep16(uint4 a) {
    uint4 r;
    if (DOT8) {
        const QNib n = nibble_form(a.x, a.y, a.z, a.w);
        r = make_uint4(n.le, n.he, n.lo, n.ho);
    } else {
        transpose4x4(a.x, a.y, a.z, a.w, r.x, r.y, r.z, r.w);
    }
    return r;
}

// 16 weights (one packed dword) against their 16 prepared activations.
template <bool DOT8>
__device__ __forceinline__ void mac16(uint32_t w, uint4 pq, int &hi, uint32_t &lo) {
    if (DOT8) {
        const uint32_t u0 = w & 0x33333333u;
        const uint32_t u1 = (w >> 2) & 0x33333333u;
        hi = sdot8(u0, pq.y, hi);
        hi = sdot8(u1, pq.w, hi);
        lo = udot8(u0, pq.x, lo);
        lo = udot8(u1, pq.z, lo);
    } else {
        hi = dot4(codes_i(w, 0), pq.x, hi);
        hi = dot4(codes_i(w, 1), pq.y, hi);
        hi = dot4(codes_i(w, 2), pq.z, hi);
        hi = dot4(codes_i(w, 3), pq.w, hi);
    }
}

// q staging for one K segment (chunks s0 .. s0 + sc - 1) of an M tile (rows m0 ..
// m0 + mcount - 1): each 16-byte piece rearranged for the dot products into LDS
// (qs, 80 bytes per 64-value chunk) and sum_k q per row added to sq.  Called by
// every thread of the workgroup between two barriers.

// From int8 q in global memory.
// Each stager has a load phase, issued before the segment's first weight loads (so
// that waiting for its data does not wait for theirs), and the staging itself.
template <int MT, bool DOT8>
struct StageQ {
    const int8_t *q;
    int K;
    struct Pre {};
    __device__ __forceinline__ Pre load(int, int) const { return Pre{}; }
    __device__ __forceinline__ void operator()(const Pre &, int s0, int sc, int m0, int mcount, int seg_chunks,
                                               uint32_t *qs, int *sq) const {
        const int tid = threadIdx.x;
        int part[MT];
        #pragma unroll
        for (int m = 0; m < MT; ++m) part[m] = 0;
        const int pieces = sc * 4;  // 16-byte pieces per row of q in this segment
        for (int idx = tid; idx < mcount * pieces; idx += blockDim.x) {
            const int m = idx / pieces, r = idx - m * pieces;
            const uint4 a = gload16(q + (size_t)(m0 + m) * K + 64 * s0 + 16 * r);
            const int c = r >> 2, d = r & 3;
            *reinterpret_cast<uint4 *>(qs + (m * seg_chunks + c) * kLdsChunkDw + 4 * d) = prep16<DOT8>(a);
            int sm = dot4(a.x, 0x01010101u, 0);
            sm = dot4(a.y, 0x01010101u, sm);
            sm = dot4(a.z, 0x01010101u, sm);
            sm = dot4(a.w, 0x01010101u, sm);
            #pragma unroll
            for (int mm = 0; mm < MT; ++mm) part[mm] += (mm == m) ? sm : 0;
        }
        #pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < mcount && part[m] != 0) atomicAdd(&sq[m], part[m]);
    }
};

// From int8 q, chunk by chunk, for weights with group-wise scales: also the sum of
// q over each 64-value chunk (sqc[m][c], plain stores), which the grouped product
// subtracts chunk by chunk (sum_k q t = sum_k q c - sum_k q within every group).
template <int MT, bool DOT8>
struct StageQChunks {
    const int8_t *q;
    int K;
    int *sqc;            // LDS, [MT][seg_chunks]
    struct Pre {};
    __device__ __forceinline__ Pre load(int, int) const { return Pre{}; }
    __device__ __forceinline__ void operator()(const Pre &, int s0, int sc, int m0, int mcount, int seg_chunks,
                                               uint32_t *qs, int *) const {
        for (int idx = threadIdx.x; idx < mcount * sc; idx += blockDim.x) {
            const int m = idx / sc, c = idx - m * sc;
            const int8_t *src = q + (size_t)(m0 + m) * K + 64 * (s0 + c);
            int sm = 0;
            #pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint4 a = gload16(src + 16 * d);
                *reinterpret_cast<uint4 *>(qs + (m * seg_chunks + c) * kLdsChunkDw + 4 * d) = prep16<DOT8>(a);
                sm = dot4(a.x, 0x01010101u, sm);
                sm = dot4(a.y, 0x01010101u, sm);
                sm = dot4(a.z, 0x01010101u, sm);
                sm = dot4(a.w, 0x01010101u, sm);
            }
            sqc[m * seg_chunks + c] = sm;
        }
    }
};

// From the bf16 activation row itself (one token, K in one segment): the
// quantization of bitnet_quant_act done in the workgroup (page chenxutan.com
// sec. 2.2, absmax_quantize): s = max|x| (integer max of the bf16 magnitude bits),
// q = rint((127 x) / s), all zero for an all-zero row.  The row scale goes to LDS
// (*s_lds) for the epilogue; q and s are also written out when q_out / s_out are set.
template <bool DOT8, int NW>
struct StageQuantize {
    static constexpr int kThreads = 64 * NW;
    static constexpr int kPre = 512 / kThreads;   // pieces per thread held in registers (K <= 8192)
    const uint16_t *x;   // [K] bf16 bits, 16-byte aligned
    int8_t *q_out;       // [K] or nullptr
    float *s_out;        // or nullptr
    float *s_lds;        // LDS
    uint32_t *red;       // LDS, one word per wavefront (NW)
    // the first kPre pieces of 16 values of each thread
    struct Pre { uint4 xr[kPre][2]; };
    __device__ __forceinline__ Pre load(int, int sc) const {
        const int pieces = sc * 4;
        Pre p;
        #pragma unroll
        for (int j = 0; j < kPre; ++j) {
            const int r = min((int)threadIdx.x + kThreads * j, pieces - 1);   // clamped duplicates leave the max as it is
            p.xr[j][0] = gload16(x + 16 * r);
            p.xr[j][1] = gload16(x + 16 * r + 8);
        }
        return p;
    }
    __device__ __forceinline__ void operator()(const Pre &pre, int, int sc, int, int, int, uint32_t *qs,
                                               int *sq) const {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int pieces = sc * 4;  // pieces of 16 values (32 bytes of x)
        uint32_t mx = 0;
        #pragma unroll
        for (int j = 0; j < kPre; ++j) mx = max(mx, max(absmax8(pre.xr[j][0]), absmax8(pre.xr[j][1])));
        for (int r = tid + 512; r < pieces; r += kThreads)
            mx = max(mx, max(absmax8(gload16(x + 16 * r)), absmax8(gload16(x + 16 * r + 8))));
        mx = wave_max_u32(mx);
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        mx = red[0];
        #pragma unroll
        for (int w = 1; w < NW; ++w) mx = max(mx, red[w]);
        const float s = bf16f(mx);
        const float inv = 1.0f / s;
        if (tid == 0) {
            *s_lds = s;
            if (s_out) *s_out = s;
        }
        int part = 0;
        auto emit = [&](int r, uint4 u0, uint4 u1) {
            uint4 a = make_uint4(0u, 0u, 0u, 0u);
            if (mx != 0) {
                const uint2 lo = qcode8(u0, s, inv), hi = qcode8(u1, s, inv);
                a = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
            if (q_out) *reinterpret_cast<uint4 *>(q_out + 16 * r) = a;
            *reinterpret_cast<uint4 *>(qs + (r >> 2) * kLdsChunkDw + 4 * (r & 3)) = prep16<DOT8>(a);
            int sm = dot4(a.x, 0x01010101u, 0);
            sm = dot4(a.y, 0x01010101u, sm);
            sm = dot4(a.z, 0x01010101u, sm);
            part += dot4(a.w, 0x01010101u, sm);
        };
        #pragma unroll
        for (int j = 0; j < kPre; ++j) {
            const int r = tid + kThreads * j;
            if (r < pieces) emit(r, pre.xr[j][0], pre.xr[j][1]);
        }
        for (int r = tid + 512; r < pieces; r += kThreads) emit(r, gload16(x + 16 * r), gload16(x + 16 * r + 8));
        if (part != 0) atomicAdd(&sq[0], part);
    }
};

// From the bf16 activation row with an RMSNorm first (page chenxutan.com sec. 3.1):
// the codes and scale of the normalized row (device_common.h, rms_*), computed in
// the workgroup from x and the gain; otherwise as StageQuantize.  The load phase
// holds one piece of 16 values (x and gain) per thread (all of K <= 64 NW 16).
template <bool DOT8, int NW>
struct StageRmsQuantize {
    static constexpr int kThreads = 64 * NW;
    const uint16_t *x;   // [K] bf16 bits, 16-byte aligned
    const float *gain;   // [K], 16-byte aligned
    float eps;
    int8_t *q_out;       // [K] or nullptr
    float *s_out;        // or nullptr
    float *s_lds;        // LDS
    double *red;         // LDS, 2 NW doubles
    struct Pre { uint4 x0, x1; float4 g0, g1, g2, g3; };
    __device__ __forceinline__ Pre load(int, int sc) const {
        const int r = min((int)threadIdx.x, sc * 4 - 1);
        Pre p;
        p.x0 = gload16(x + 16 * r);
        p.x1 = gload16(x + 16 * r + 8);
        const float4 *g = reinterpret_cast<const float4 *>(gain + 16 * r);
        p.g0 = g[0]; p.g1 = g[1]; p.g2 = g[2]; p.g3 = g[3];
        return p;
    }
    __device__ __forceinline__ void operator()(const Pre &pre, int, int sc, int, int, int, uint32_t *qs,
                                               int *sq) const {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int pieces = sc * 4;
        auto gain4 = [&](int r, float4 (&g)[4]) {
            const float4 *gp = reinterpret_cast<const float4 *>(gain + 16 * r);
            g[0] = gp[0]; g[1] = gp[1]; g[2] = gp[2]; g[3] = gp[3];
        };
        double mz = 0.0, ss = 0.0;
        if (tid < pieces) {
            rms_acc8(pre.x0, pre.g0, pre.g1, mz, ss);
            rms_acc8(pre.x1, pre.g2, pre.g3, mz, ss);
        }
        for (int r = tid + kThreads; r < pieces; r += kThreads) {
            float4 g[4];
            gain4(r, g);
            rms_acc8(gload16(x + 16 * r), g[0], g[1], mz, ss);
            rms_acc8(gload16(x + 16 * r + 8), g[2], g[3], mz, ss);
        }
        mz = wave_max_f64(mz);
        ss = wave_sum_f64(ss);
        if (lane == 0) { red[wave] = mz; red[NW + wave] = ss; }
        __syncthreads();
        mz = red[0];
        ss = red[NW];
        #pragma unroll
        for (int w = 1; w < NW; ++w) { mz = fmax(mz, red[w]); ss += red[NW + w]; }
        const float s = rms_scale(mz, ss, 64 * sc, eps);
        const double c = mz > 0.0 ? 127.0 / mz : 0.0;
        if (tid == 0) {
            *s_lds = s;
            if (s_out) *s_out = s;
        }
        int part = 0;
        auto emit = [&](int r, uint4 u0, uint4 u1, float4 g0, float4 g1, float4 g2, float4 g3) {
            uint4 a = make_uint4(0u, 0u, 0u, 0u);
            if (mz > 0.0) {
                const uint2 lo = rms_code8(u0, g0, g1, c, mz), hi = rms_code8(u1, g2, g3, c, mz);
                a = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
            if (q_out) *reinterpret_cast<uint4 *>(q_out + 16 * r) = a;
            *reinterpret_cast<uint4 *>(qs + (r >> 2) * kLdsChunkDw + 4 * (r & 3)) = prep16<DOT8>(a);
            int sm = dot4(a.x, 0x01010101u, 0);
            sm = dot4(a.y, 0x01010101u, sm);
            sm = dot4(a.z, 0x01010101u, sm);
            part += dot4(a.w, 0x01010101u, sm);
        };
        if (tid < pieces) emit(tid, pre.x0, pre.x1, pre.g0, pre.g1, pre.g2, pre.g3);
        for (int r = tid + kThreads; r < pieces; r += kThreads) {
            float4 g[4];
            gain4(r, g);
            emit(r, gload16(x + 16 * r), gload16(x + 16 * r + 8), g[0], g[1], g[2], g[3]);
        }
        if (part != 0) atomicAdd(&sq[0], part);
    }
};

// From an fp32 activation row (such as the SwiGLU output that feeds a down
// projection, page chenxutan.com sec. 3.1): the same absmax quantization (sec. 2.2)
// of fp32 values, s = max|x| (integer max of the magnitude bits), codes by
// qcode_f32; otherwise as StageQuantize.  The load phase holds one piece of 16
// values per thread; the thread's second piece is held from the max to the codes,
// later pieces (K > 64 NW 32) are read again.
template <bool DOT8, int NW>
struct StageQuantizeF32 {
    static constexpr int kThreads = 64 * NW;
    const float *x;      // [K] fp32, 16-byte aligned
    int8_t *q_out;       // [K] or nullptr
    float *s_out;        // or nullptr
    float *s_lds;        // LDS
    uint32_t *red;       // LDS, one word per wavefront (NW)
    struct Pre { float4 v[4]; };
    __device__ __forceinline__ Pre load(int, int sc) const {
        const int r = min((int)threadIdx.x, sc * 4 - 1);   // a clamped duplicate leaves the max as it is
        const float4 *p = reinterpret_cast<const float4 *>(x + 16 * r);
        Pre pre;
        #pragma unroll
        for (int i = 0; i < 4; ++i) pre.v[i] = p[i];
        return pre;
    }
    __device__ __forceinline__ void operator()(const Pre &pre, int, int sc, int, int, int, uint32_t *qs,
                                               int *sq) const {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int pieces = sc * 4;
        const float4 *xv = reinterpret_cast<const float4 *>(x);
        const int r1 = tid + kThreads;
        float4 v1[4];
        #pragma unroll
        for (int i = 0; i < 4; ++i) v1[i] = xv[4 * min(r1, pieces - 1) + i];
        uint32_t mx = max(absmax8_f32(pre.v[0], pre.v[1]), absmax8_f32(pre.v[2], pre.v[3]));
        mx = max(mx, max(absmax8_f32(v1[0], v1[1]), absmax8_f32(v1[2], v1[3])));
        for (int r = tid + 2 * kThreads; r < pieces; r += kThreads)
            mx = max(mx, max(absmax8_f32(xv[4 * r], xv[4 * r + 1]), absmax8_f32(xv[4 * r + 2], xv[4 * r + 3])));
        mx = wave_max_u32(mx);
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        mx = red[0];
        #pragma unroll
        for (int w = 1; w < NW; ++w) mx = max(mx, red[w]);
        const float s = __uint_as_float(mx);
        const float inv = 1.0f / s;
        if (tid == 0) {
            *s_lds = s;
            if (s_out) *s_out = s;
        }
        int part = 0;
        auto emit = [&](int r, const float4 (&v)[4]) {
            uint4 b = make_uint4(0u, 0u, 0u, 0u);
            if (mx != 0) {
                const float lo[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
                const float hi[8] = {v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
                const uint2 cl = qcode8_f32(lo, s, inv), ch = qcode8_f32(hi, s, inv);
                b = make_uint4(cl.x, cl.y, ch.x, ch.y);
            }
            if (q_out) *reinterpret_cast<uint4 *>(q_out + 16 * r) = b;
            *reinterpret_cast<uint4 *>(qs + (r >> 2) * kLdsChunkDw + 4 * (r & 3)) = prep16<DOT8>(b);
            int sm = dot4(b.x, 0x01010101u, 0);
            sm = dot4(b.y, 0x01010101u, sm);
            sm = dot4(b.z, 0x01010101u, sm);
            part += dot4(b.w, 0x01010101u, sm);
        };
        if (tid < pieces) emit(tid, pre.v);
        if (r1 < pieces) emit(r1, v1);
        for (int r = tid + 2 * kThreads; r < pieces; r += kThreads) {
            const float4 v[4] = {xv[4 * r], xv[4 * r + 1], xv[4 * r + 2], xv[4 * r + 3]};
            emit(r, v);
        }
        if (part != 0) atomicAdd(&sq[0], part);
    }
};

// s_x is not restrict-qualified: in the fused kernels it is the LDS word the stager
// writes through its own pointer, and its reads must stay after the staging.
// GRP: the weights have group-wise scales (out.w_group = G, a multiple of 64 below K):
// each chunk's integer partial, less its sum of q (sqc), is scaled by its group's
// s_w[row][k / G] and summed in float64 (kslices == 1 only).
// PAIR: the gate (packed, s_w) and up (packed2, s_w2) projections of a SwiGLU
// feed-forward part (page chenxutan.com sec. 3.1) against the same row of q
// (kslices == 1, MT == 1): the first NW / 2 waves take rows [row_base, row_base +
// 4 NW RG) of gate, the others the same rows of up; the epilogue meets the two fp32
// outputs of each row in LDS (ypair, 8 NW RG floats) and writes
// a = fp32(silu(y_gate) y_up) (device_common.h, swiglu_value) to out.y.
template <int MT, int RG, bool DOT8, bool NT, int NW, class Stage, bool GRP = false, bool PAIR = false,
          int PI = BITNET_GEMV_PREISSUE>
__device__ __forceinline__ void gemv_lds_tile(const Stage &stage, const float *s_x,
                                              const uint8_t *__restrict__ packed,
                                              const float *__restrict__ s_w, int M, int N, int K,
                                              const OutSpec &out, int32_t *__restrict__ acc_out,
                                              int row_base, int m0, int kslices, int seg_chunks,
                                              uint32_t *qs, int *sq, int *red, const int *sqc = nullptr,
                                              const uint8_t *__restrict__ packed2 = nullptr,
                                              const float *__restrict__ s_w2 = nullptr, float *ypair = nullptr) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l8 = lane & 7, rs = lane >> 3;
    const int C = K >> 6;
    const int KB = K >> 2;
    const int mcount = min(MT, M - m0);

    // wave -> (row set, K slice of every segment); PAIR: wave -> (matrix, row set)
    const int half = PAIR && wave >= NW / 2 ? 1 : 0;
    const int rowset = PAIR ? wave - half * (NW / 2) : wave / kslices;
    const int slice = PAIR ? 0 : wave - rowset * kslices;
    const int row0 = row_base + rowset * 8 * RG;
    if (PAIR && half) {
        packed = packed2;
        s_w = s_w2;
    }

    int hi[RG][MT];
    uint32_t lo[RG][MT];
    double facc[RG][MT];       // GRP: sum over chunks of partial x group scale
    const uint8_t *prow[RG];
    const float *srow[RG];     // GRP: the row's group scales
    const int G = GRP ? out.w_group : 1, ng = GRP ? K / G : 1;
    #pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int r = row0 + 8 * g + rs;
        prow[g] = packed + (size_t)(r < N ? r : 0) * KB;   // rows past N read row 0, discarded
        srow[g] = s_w + (size_t)(r < N ? r : 0) * ng;
        #pragma unroll
        for (int m = 0; m < MT; ++m) { hi[g][m] = 0; lo[g][m] = 0u; facc[g][m] = 0.0; }
    }
    if (tid < MT) sq[tid] = 0;
    // the per-tensor weight scale, read before the weight stream so that its latency
    // is not paid after the last chunk
    const float sw = *(const __attribute__((address_space(4))) float *)s_w;   // read-only here: scalar load
    // chunk offset of this lane's rows within their 128-byte line (the same for all
    // RG groups: their rows differ by multiples of 8)
    const int line_off = (int)((((uint32_t)(row0 + rs) & 7u) * ((uint32_t)(KB >> 4) & 7u)) & 7u);

    // K is walked in segments of seg_chunks 64-weight chunks; the q tile of a segment
    // (MT rows) is what LDS holds, so any K and M tile fit the LDS budget.
    for (int s0 = 0; s0 < C; s0 += seg_chunks) {
        const int sc = min(seg_chunks, C - s0);
        const int cb = s0 + (int)(((int64_t)sc * slice) / kslices);
        const int ce = s0 + (int)(((int64_t)sc * (slice + 1)) / kslices);

        // Step t of the octet reads one aligned 128-byte line of its row: lane l8 takes
        // 16-byte slot l8 of line t, i.e. chunk c0 + 8 t + l8 with c0 = the chunk at
        // the start of the line holding chunk cb (rows may start mid-line: for
        // K = 6912 odd rows start 64 bytes into a line).  Lanes whose chunk falls
        // outside [cb, ce) load a clamped in-range chunk and use all-zero codes, which
        // add nothing; an unaligned start costs one more step.  Two register buffers
        // alternate so that the loads of step t + 1 are in flight during step t.
        const int c0 = ((line_off + cb) & ~7) - line_off;
        const bool aligned = ((KB >> 4) & 7) == 0 && (cb & 7) == 0;
        // a wave whose rows all lie past N loads (clamped, unused) but computes nothing
        const int T = row0 < N ? ((ce - cb + 7) >> 3) + (aligned ? 0 : 1) : 0;
        const int clast = min(max(ce - 1, cb), C - 1);   // in range even for an empty slice
        struct WBuf { uint4 w[RG]; float s[RG]; };   // s: GRP group scales of the chunk
        WBuf bufA, bufB;
        auto issue = [&](WBuf &b, int t) {
            const int cc = min(max(c0 + l8 + 8 * t, cb), clast);
            #pragma unroll
            for (int g = 0; g < RG; ++g) b.w[g] = load_weights<NT>(prow[g] + 16 * cc);
            if (GRP) {
                #pragma unroll
                for (int g = 0; g < RG; ++g) b.s[g] = srow[g][(64 * cc) / G];
            }
        };
        auto consume = [&](const WBuf &b, int t) {
            const int craw = c0 + l8 + 8 * t;
            const bool valid = craw >= cb && craw < ce;
            const int cc = min(max(craw, cb), clast) - s0;
            #pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mcount) {
                    const uint32_t *qc = qs + (m * seg_chunks + cc) * kLdsChunkDw;
                    int hc[RG];
                    uint32_t lc[RG];
                    #pragma unroll
                    for (int g = 0; g < RG; ++g) { hc[g] = 0; lc[g] = 0u; }
                    #pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint4 pq = *reinterpret_cast<const uint4 *>(qc + 4 * d);
                        #pragma unroll
                        for (int g = 0; g < RG; ++g) {
                            uint32_t wd = d == 0 ? b.w[g].x : d == 1 ? b.w[g].y : d == 2 ? b.w[g].z : b.w[g].w;
                            wd = valid ? wd : 0u;
                            if (GRP) mac16<DOT8>(wd, pq, hc[g], lc[g]);
                            else mac16<DOT8>(wd, pq, hi[g][m], lo[g][m]);
                        }
                    }
                    if (GRP) {
                        const int sqv = valid ? sqc[m * seg_chunks + cc] : 0;
                        #pragma unroll
                        for (int g = 0; g < RG; ++g) {
                            const int p = (DOT8 ? 16 * hc[g] + (int)lc[g] : hc[g]) - sqv;   // |p| <= 64 * 127
                            hi[g][m] += p;
                            facc[g][m] += (double)p * (double)b.s[g];
                        }
                    }
                }
            }
        };
        // The stager's loads go out first, then the segment's first weight loads, so
        // that the staging waits only for its own data while the weights are in flight.
        // Both issues are unconditional (a step past the last reads a clamped in-range
        // chunk and is never consumed): a branch here would make the compiler's wait
        // for the stager's data also wait for these loads.
        const typename Stage::Pre pre = stage.load(s0, sc);
        issue(bufA, 0);
        if (PI > 1) issue(bufB, 1);

        // ---- stage the segment of the M tile of q, rearranged, and its row sums
        __syncthreads();   // previous segment's LDS reads done; sq initialised
        stage(pre, s0, sc, m0, mcount, seg_chunks, qs, sq);
        __syncthreads();

        // Pairs of chunks with no branch inside the loop body, so that the compiler
        // waits for exactly the older buffer's loads; the last one or two chunks are
        // peeled (a uniform branch outside the loop).
        if (T > 0) {
            const int T2 = (T + 1) & ~1;
            if (PI > 1) {
                // steps t and t + 1 are in flight at the top of every iteration
                int t = 0;
                for (; t + 3 < T; t += 2) {
                    consume(bufA, t);
                    issue(bufA, t + 2);
                    consume(bufB, t + 1);
                    issue(bufB, t + 3);
                }
                if (T - t == 3) {
                    consume(bufA, t);
                    issue(bufA, t + 2);
                    consume(bufB, t + 1);
                    consume(bufA, t + 2);
                } else if (T - t == 2) {
                    consume(bufA, t);
                    consume(bufB, t + 1);
                } else {
                    consume(bufA, t);
                }
            } else {
                for (int t = 0; t < T2 - 2; t += 2) {
                    issue(bufB, t + 1);
                    consume(bufA, t);
                    issue(bufA, t + 2);
                    consume(bufB, t + 1);
                }
                if (T2 == T) {
                    issue(bufB, T - 1);
                    consume(bufA, T - 2);
                    consume(bufB, T - 1);
                } else {
                    consume(bufA, T - 1);
                }
            }
        }
    }

    if (GRP) {
        // hi holds the exact integer sum (sq already subtracted chunk by chunk); facc
        // the scaled sum: y = fp32((sum_g acc_g s_g) s_x / 127 (+ bias))
        #pragma unroll
        for (int m = 0; m < MT; ++m) {
            #pragma unroll
            for (int g = 0; g < RG; ++g) {
                const int a = octet_sum(hi[g][m]);
                const double f = octet_sum_f64(facc[g][m]);
                const int r = row0 + 8 * g + rs;
                if (m < mcount && r < N && l8 == (m & 7)) {
                    const size_t o = (size_t)(m0 + m) * N + r;
                    double v = (f * (double)s_x[m0 + m]) / 127.0;
                    if (out.bias) v += (double)out.bias[r];
                    store_y(out, o, v);
                    if (acc_out) acc_out[o] = a;
                }
            }
        }
        return;
    }
    int acc[RG][MT];
    #pragma unroll
    for (int g = 0; g < RG; ++g) {
        #pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[g][m] = octet_sum(DOT8 ? 16 * hi[g][m] + (int)lo[g][m] : hi[g][m]);
    }

    if (PAIR) {
        constexpr int kHalfRows = (NW / 2) * 8 * RG;
        const double cm = rescale_factor(s_x[m0], sw);
        if (l8 == 0) {
            #pragma unroll
            for (int g = 0; g < RG; ++g)
                ypair[half * kHalfRows + rowset * 8 * RG + 8 * g + rs] = rescale(acc[g][0] - sq[0], cm);
        }
        __syncthreads();
        const int r = row_base + tid;
        if (tid < kHalfRows && r < N) store_y(out, (size_t)m0 * N + r, (double)swiglu_value(ypair[tid], ypair[kHalfRows + tid]));
        return;
    }
    if (BITNET_GEMV_WG_STORE && MT == 1 && kslices == 1) {
        // one token: the row sums of all wavefronts meet in red (LDS) and wavefront 0
        // stores the workgroup's rows, consecutive lanes on consecutive rows; the other
        // wavefronts end without stores of their own to wait for
        if (l8 == 0) {
            #pragma unroll
            for (int g = 0; g < RG; ++g) red[wave * 8 * RG + 8 * g + rs] = acc[g][0];
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (wave != 0 || mcount <= 0) return;
        const double cm = rescale_factor(s_x[m0], sw);
        #pragma unroll
        for (int i = 0; i < (NW * 8 * RG + 63) / 64; ++i) {
            const int j = 64 * i + lane;
            const int r = row_base + j;
            if (j < NW * 8 * RG && r < N) {
                const size_t o = (size_t)m0 * N + r;
                const int a = red[j] - sq[0];
                put_y(out, o, r, a, col_factor(out, s_w, r, s_x[m0], cm));
                if (acc_out) acc_out[o] = a;
            }
        }
        return;
    }
    if (kslices == 1) {
        #pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= mcount) continue;
            const double cm = rescale_factor(s_x[m0 + m], sw);
            const int sqm = sq[m];
            #pragma unroll
            for (int g = 0; g < RG; ++g) {
                const int r = row0 + 8 * g + rs;
                if (r < N && l8 == (m & 7)) {
                    const size_t o = (size_t)(m0 + m) * N + r;
                    const int a = acc[g][m] - sqm;
                    put_y(out, o, r, a, col_factor(out, s_w, r, s_x[m0 + m], cm));
                    if (acc_out) acc_out[o] = a;
                }
            }
        }
        return;
    }
    constexpr int R = 8 * RG;
    if (l8 == 0) {
        #pragma unroll
        for (int g = 0; g < RG; ++g) {
            #pragma unroll
            for (int m = 0; m < MT; ++m) red[(wave * R + 8 * g + rs) * MT + m] = acc[g][m];
        }
    }
    __syncthreads();
    const int rowsets = NW / kslices;
    for (int idx = tid; idx < rowsets * R * MT; idx += blockDim.x) {
        const int rsi = idx / (R * MT), rem = idx - rsi * R * MT;
        const int rr = rem / MT, m = rem - rr * MT;
        const int r = row_base + rsi * R + rr;
        if (r >= N || m >= mcount) continue;
        int s = -sq[m];
        for (int w = 0; w < kslices; ++w) s += red[((rsi * kslices + w) * R + rr) * MT + m];
        const size_t o = (size_t)(m0 + m) * N + r;
        put_y(out, o, r, s, col_factor(out, s_w, r, s_x[m0 + m], rescale_factor(s_x[m0 + m], sw)));
        if (acc_out) acc_out[o] = s;
    }
}

template <int MT, int RG, bool DOT8, bool GRP>
__global__ __launch_bounds__(256) void gemv_lds_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s_x, const uint8_t *__restrict__ packed,
    const float *__restrict__ s_w, int M, int N, int K, const OutSpec out,
    int32_t *__restrict__ acc_out, int kslices, int seg_chunks) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    __shared__ int sq[MT];
    __shared__ int red[4 * 8 * RG * MT];
    const int rows_per_block = (4 / kslices) * 8 * RG;
    if (GRP) {
        // the chunk sums of q follow the staged q in the dynamic LDS
        int *sqc = reinterpret_cast<int *>(dyn + MT * seg_chunks * kLdsChunkDw);
        gemv_lds_tile<MT, RG, DOT8, BITNET_GEMV_NT != 0, 4, StageQChunks<MT, DOT8>, true>(
            StageQChunks<MT, DOT8>{q, K, sqc}, s_x, packed, s_w, M, N, K, out, acc_out, blockIdx.x * rows_per_block,
            blockIdx.y * MT, 1, seg_chunks, dyn, sq, red, sqc);
    } else {
        gemv_lds_tile<MT, RG, DOT8, BITNET_GEMV_NT != 0, 4>(StageQ<MT, DOT8>{q, K}, s_x, packed, s_w, M, N, K, out,
                                                         acc_out, blockIdx.x * rows_per_block, blockIdx.y * MT,
                                                         kslices, seg_chunks, dyn, sq, red);
    }
}

// K segment length in 64-weight chunks for an M tile of mt rows: the whole of K when
// its staged q fits the LDS budget, else the fewest segments of equal size, each a
// multiple of 8 chunks (one per lane of an octet).
// dw: LDS dwords per staged chunk (kLdsChunkDw, or one more with group-wise scales,
// which also keep each chunk's sum of q).
__host__ __device__ __forceinline__ int segment_chunks(int C, int mt, int dw = kLdsChunkDw) {
    const int max_seg = (kLdsBudget / (mt * dw * 4)) & ~7;
    if (C <= max_seg) return C;
    const int nseg = (C + max_seg - 1) / max_seg;
    return (((C + nseg - 1) / nseg) + 7) & ~7;
}

// Grouped decode: 4 wavefronts per block, block -> (descriptor, row block, M tile)
// through the plan's block table; staged-q LDS size comes from the plan header.
constexpr int kGroupedRG = BITNET_GROUPED_RG;
constexpr int kGroupedMT = 1;   // tokens per workgroup of the plain grouped GEMV

// GRP: the plan has problems with group-wise weight scales (descriptor w_group below
// K), which take the grouped tile; plans without them use the kernel without it.
template <bool GRP, int MT>
__global__ __launch_bounds__(256) void gemv_grouped_kernel(const uint8_t *__restrict__ plan) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    __shared__ int sq[MT];
    __shared__ int red[4 * 8 * kGroupedRG * MT];
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[blockIdx.x];
    const LinearDescDev d = reinterpret_cast<const LinearDescDev *>(plan + h->desc_offset)[e.desc];
    const int rows = 4 * 8 * kGroupedRG;
    const int rowblocks = (d.N + rows - 1) / rows;
    const int rb = (int)(e.local % rowblocks), mt = (int)(e.local / rowblocks);
    const OutSpec out = d.out();
    constexpr bool D8 = BITNET_GROUPED_DOT8 != 0, NTL = BITNET_GEMV_NT != 0;
    if (GRP && d.w_group > 0 && d.w_group < d.K) {
        const int seg = segment_chunks(d.K >> 6, MT, kLdsChunkDw + 1);
        int *sqc = reinterpret_cast<int *>(dyn + MT * seg * kLdsChunkDw);
        gemv_lds_tile<MT, kGroupedRG, D8, NTL, 4, StageQChunks<MT, D8>, true>(
            StageQChunks<MT, D8>{d.q, d.K, sqc}, d.s_x, d.packed, d.s_w, d.M, d.N, d.K, out, d.acc, rb * rows,
            mt * MT, 1, seg, dyn, sq, red, sqc);
    } else {
        gemv_lds_tile<MT, kGroupedRG, D8, NTL, 4>(
            StageQ<MT, D8>{d.q, d.K}, d.s_x, d.packed, d.s_w, d.M, d.N, d.K, out, d.acc, rb * rows,
            mt * MT, 1, segment_chunks(d.K >> 6, MT), dyn, sq, red);
    }
}

// Fused grouped decode: the same work items, with the activation quantization of
// each problem's token row done by every workgroup of that problem in its q
// staging step (one segment, so the row max covers the whole row).  The workgroup of
// row block 0 also writes q and s_x out when the descriptor asks for them.
constexpr int kFusedNW = BITNET_FUSED_NW;
constexpr int kFusedRG = BITNET_FUSED_RG;
constexpr int kFusedPI = BITNET_FUSED_PREISSUE;

// PRO: the mask of paths the plan's problems use (kFusedProNorm: an RMSNorm;
// kFusedProSwiglu: fp32 input rows and gate / up pairs with the SwiGLU epilogue);
// each problem takes the stager and epilogue its descriptor asks for, and a kernel
// holds only the paths of its mask (fewer registers without them).  Every wavefront
// keeps two steps of weight loads in flight, the first two issued before the q
// staging.  Waves per SIMD: at least 5 for the plain kernel (no spills; fewer bytes in
// flight per CU than at 6 with one step pre-issued, so the x row waits less behind
// the weight stream: 82.0 -> 80.7 us per decode step), at least 4 for the others.
// (The output spec is built in each call, not kept in a named local, which costs
// registers here.)
template <int PRO>
__global__ __launch_bounds__(64 * kFusedNW) __attribute__((amdgpu_waves_per_eu(PRO == 0 ? 5 : 4)))
void gemv_fused_grouped_kernel(const uint8_t *__restrict__ plan) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    __shared__ int sq[1];
    __shared__ int red[kFusedNW * 8 * kFusedRG];
    __shared__ uint32_t qred[kFusedNW];
    __shared__ double dred[2 * kFusedNW];
    __shared__ float s_lds;
    __shared__ float ypair[(PRO & kFusedProSwiglu) ? kFusedNW * 8 * kFusedRG : 1];
    const PlanHeader *h = reinterpret_cast<const PlanHeader *>(plan);
    auto entry = [&](uint32_t b) {
        const BlockEntry e = reinterpret_cast<const BlockEntry *>(plan + h->table_offset)[b];
        const FusedDescDev d = reinterpret_cast<const FusedDescDev *>(plan + h->desc_offset)[e.desc];
        const int rows = kFusedNW * 8 * kFusedRG;
        const bool first = e.local == 0;
        constexpr bool D8 = BITNET_GROUPED_DOT8 != 0, NTL = BITNET_GEMV_NT != 0;
        // a gate / up pair covers half the rows per workgroup (each row twice)
        const bool pair = (PRO & kFusedProSwiglu) && d.packed2;
        const int row_base = (int)e.local * (pair ? rows / 2 : rows);
        // the tile for a stager: a gate / up pair (SwiGLU epilogue) or one matrix
        auto tile = [&](const auto &stage, bool as_pair) {
            using S = std::decay_t<decltype(stage)>;
            if ((PRO & kFusedProSwiglu) && as_pair)
                gemv_lds_tile<1, kFusedRG, D8, NTL, kFusedNW, S, false, true, kFusedPI>(
                    stage, &s_lds, d.packed, d.s_w, 1, d.N, d.K, OutSpec{d.y, nullptr, d.bf16, 0}, nullptr, row_base, 0, 1,
                    d.K >> 6, dyn, sq, red, nullptr, d.packed2, d.s_w2, ypair);
            else
                gemv_lds_tile<1, kFusedRG, D8, NTL, kFusedNW, S, false, false, kFusedPI>(stage, &s_lds, d.packed, d.s_w, 1, d.N, d.K,
                                                                 OutSpec{d.y, d.bias, d.bf16, 0}, d.acc, row_base, 0, 1,
                                                                 d.K >> 6, dyn, sq, red);
        };
        int8_t *q_out = first ? d.q : nullptr;
        float *s_out = first ? d.s_x : nullptr;
        if ((PRO & kFusedProNorm) && d.gain)
            tile(StageRmsQuantize<D8, kFusedNW>{d.x, d.gain, d.eps, q_out, s_out, &s_lds, dred}, pair);
        else if ((PRO & kFusedProSwiglu) && d.xf)
            tile(StageQuantizeF32<D8, kFusedNW>{d.xf, q_out, s_out, &s_lds, qred}, false);
        else
            tile(StageQuantize<D8, kFusedNW>{d.x, q_out, s_out, &s_lds, qred}, pair);
    };
    if (BITNET_FUSED_PERSIST == 0) {
        // one entry per workgroup and no loop: with memory operations of a previous
        // entry pending at a loop head, the compiler's waits in the staging become
        // waits for everything, weight loads included
        entry(blockIdx.x);
    } else {
        for (uint32_t b = blockIdx.x; b < h->total_blocks; b += gridDim.x) {
            entry(b);
            __builtin_amdgcn_s_waitcnt(0);   // nothing pending at the loop head
            __syncthreads();                  // LDS of this entry read by all before the next
        }
    }
}

// Longest K whose q fits one LDS segment of the grouped GEMV.
int64_t gemv_fused_max_k() { return 64 * (int64_t)((kLdsBudget / (kLdsChunkDw * 4)) & ~7); }

hipError_t launch_gemv_fused_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, uint32_t pro,
                                     hipStream_t st) {
    if (BITNET_FUSED_PERSIST > 0) blocks = std::min<uint32_t>(blocks, BITNET_FUSED_PERSIST);
    const uint8_t *p = reinterpret_cast<const uint8_t *>(plan_dev);
    const dim3 grid(blocks), block(64 * kFusedNW);
    switch (pro) {
        case 0: gemv_fused_grouped_kernel<0><<<grid, block, lds_bytes, st>>>(p); break;
        case kFusedProNorm: gemv_fused_grouped_kernel<kFusedProNorm><<<grid, block, lds_bytes, st>>>(p); break;
        case kFusedProSwiglu: gemv_fused_grouped_kernel<kFusedProSwiglu><<<grid, block, lds_bytes, st>>>(p); break;
        case kFusedProMask: gemv_fused_grouped_kernel<kFusedProMask><<<grid, block, lds_bytes, st>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

uint32_t gemv_grouped_rows_per_block() { return 4 * 8 * kGroupedRG; }
uint32_t gemv_fused_rows_per_block() { return kFusedNW * 8 * kFusedRG; }
uint32_t gemv_fused_threads() { return 64 * kFusedNW; }
uint32_t gemv_grouped_threads() { return 256; }
uint32_t gemv_grouped_lds_bytes(int64_t K, bool grp, int mt) {
    const int dw = kLdsChunkDw + (grp ? 1 : 0);
    return (uint32_t)(mt * segment_chunks((int)(K / 64), mt, dw) * dw * 4);
}

template <int MT, int RG, bool DOT8, bool GRP>
static hipError_t launch_lds(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                             int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    const int C = (int)(K / 64);
    const unsigned gy = (unsigned)((M + MT - 1) / MT);
    // more K slices per row set until the launch has >= 2 workgroups per CU,
    // keeping at least 2 chunk iterations per lane (one slice with group scales)
    int ks = 1;
    auto blocks = [&](int k) { return (int64_t)((N + (4 / k) * 8 * RG - 1) / ((4 / k) * 8 * RG)) * gy; };
    while (!GRP && ks < 4 && blocks(ks) < 512 && C / (8 * ks * 2) >= 2) ks *= 2;
    const unsigned gx = (unsigned)((N + (4 / ks) * 8 * RG - 1) / ((4 / ks) * 8 * RG));
    // with group scales each staged chunk also keeps its sum of q (one more dword)
    const int per_chunk_dw = kLdsChunkDw + (GRP ? 1 : 0);
    int seg = C;
    const int max_seg = (kLdsBudget / (MT * per_chunk_dw * 4)) & ~7;
    if (C > max_seg) {
        const int nseg = (C + max_seg - 1) / max_seg;
        seg = (((C + nseg - 1) / nseg) + 7) & ~7;
    }
    const size_t lds = (size_t)MT * seg * per_chunk_dw * 4;
    gemv_lds_kernel<MT, RG, DOT8, GRP><<<dim3(gx, gy), dim3(256), lds, st>>>(q, s_x, packed, s_w, (int)M, (int)N,
                                                                             (int)K, y, acc, ks, seg);
    return hipGetLastError();
}

constexpr int64_t kGemvTallN = 16384;

template <bool GRP>
static hipError_t launch_gemv_mt(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                                 int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    const bool d8 = BITNET_GROUPED_DOT8 != 0;
    // one token: 4 rows per octet for tall matrices (fewer LDS reads and less loop
    // work per weight), BITNET_GEMV1_RG otherwise (more workgroups for a small N) and
    // with group scales (whose tile needs more registers per row)
    if (!GRP && M == 1 && N >= kGemvTallN)
        return launch_lds<1, 4, d8, GRP>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    if (M == 1) return launch_lds<1, BITNET_GEMV1_RG, d8, GRP>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    if (M == 2) return launch_lds<2, 2, d8, GRP>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    if (M <= 4) return launch_lds<4, 2, d8, GRP>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    return launch_lds<8, 2, d8, GRP>(q, s_x, packed, s_w, M, N, K, y, acc, st);
}

hipError_t launch_gemv(const int8_t *q, const float *s_x, const uint8_t *packed, const float *s_w,
                       int64_t M, int64_t N, int64_t K, const OutSpec &y, int32_t *acc, hipStream_t st) {
    // group-wise weight scales (a group smaller than the row) take the grouped path;
    // one scale per tensor or per output channel only changes the epilogue
    if (y.w_group > 0 && y.w_group < K) return launch_gemv_mt<true>(q, s_x, packed, s_w, M, N, K, y, acc, st);
    return launch_gemv_mt<false>(q, s_x, packed, s_w, M, N, K, y, acc, st);
}

hipError_t launch_gemv_grouped(const void *plan_dev, uint32_t blocks, uint32_t lds_bytes, uint32_t variant,
                               hipStream_t st) {
    const uint8_t *p = reinterpret_cast<const uint8_t *>(plan_dev);
    if (variant == kVariantGemvGroupsMT)
        gemv_grouped_kernel<true, kGemvGroupsMT><<<dim3(blocks), dim3(256), lds_bytes, st>>>(p);
    else if (variant == kVariantGemvGroups)
        gemv_grouped_kernel<true, kGroupedMT><<<dim3(blocks), dim3(256), lds_bytes, st>>>(p);
    else
        gemv_grouped_kernel<false, kGroupedMT><<<dim3(blocks), dim3(256), lds_bytes, st>>>(p);
    return hipGetLastError();
}

}  // namespace bitnet
