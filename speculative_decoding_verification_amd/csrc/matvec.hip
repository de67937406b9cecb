// matvec.hip - the verification projection (a3), its fused producer
// epilogue (a4) and the output head with fused argmax (a6, a9).
//
// One weight stream serves all M positions ("Inside OpenJet Engine: making
// speculative decoding pay", section "One GPU launch for a speculative
// cycle": weight reads serve multiple verification positions, and
// activation loads are reused across weight rows).
//
// Work mapping (one 256-thread workgroup = 4 waves per row tile):
//  * The K axis is cut into 32-element sub-blocks.  A group of g lanes
//    (g = 32 or 16, fixed by K alone) shares one row; lane j of the group
//    takes sub-blocks j, j+g, j+2g, ... so g lanes read g consecutive 16-byte
//    records of the row: one contiguous, aligned run per group.
//  * Each lane carries R = 4 rows (row slots).  The activations of its
//    sub-block are read from LDS once per step and reused for all R rows;
//    the weights are read from HBM once and reused for all M positions.
//  * Integer block sums come from v_dot4 (exact); the fp32 combine of a
//    block is a fixed sequence of operations per (row, position); a lane
//    accumulates its blocks in increasing order, then the g lanes of a group
//    are combined by a butterfly.  None of this depends on M, so a row's
//    result is bit-identical whatever else is in the batch.
//  * Weights for the next step are loaded while the current step computes.
#include <algorithm>

#include "sv_internal.h"

namespace sv {

constexpr int kThreads = 256;
constexpr int kR = 4;
constexpr int kLdsBudget = 64 * 1024;

struct MvArgs {
    const uint8_t *w[3];
    int n_w;
    int64_t N;      // output rows (tile space)
    int64_t K;      // input features
    int64_t wrows;  // rows of the stored matrix (stream strides)
    size_t o1, o2, o3;
    const int32_t *row_ids;
    const int8_t *aq;
    const float *ad;
    const int32_t *as16;
    const float *in_parts;
    int n_parts;
    float eps;
    float *y[3];
    int ep_mode, ep_src;
    const float *gamma;
    int8_t *oq;
    float *od;
    int32_t *os16;
    float *osumsq;
    unsigned long long *argmax;
    int chunk_sub;
    int n_tiles;
};

// Bytes of LDS per position per staged sub-block: 32 codes, fp32 scale, and
// 8 bytes of per-format activation sums.
constexpr int kActRec = 32 + 4 + 8;

template <int QT>
struct WRaw;
template <>
struct WRaw<SV_Q8_0> {
    uint4 q0, q1;
    uint32_t d;
};
template <>
struct WRaw<SV_Q4_K> {
    uint4 q, h;
};
template <>
struct WRaw<SV_Q6_K> {
    uint4 l;
    uint2 h;
    uint32_t sc, d;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const uint8_t *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const uint8_t *p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(v.x, v.y);
}

template <int QT>
__device__ __forceinline__ void load_w(WRaw<QT> &r, const uint8_t *__restrict__ w, const MvArgs &a, int64_t row,
                                       int64_t s) {
    const int64_t nsub = a.K >> 5;
    if constexpr (QT == SV_Q8_0) {
        r.q0 = ld_stream16(w + row * a.K + s * 32);
        r.q1 = ld_stream16(w + row * a.K + s * 32 + 16);
        r.d = *reinterpret_cast<const uint16_t *>(w + a.o1 + (row * nsub + s) * 2);
    } else if constexpr (QT == SV_Q4_K) {
        r.q = ld_stream16(w + (row * nsub + s) * 16);
        r.h = *reinterpret_cast<const uint4 *>(w + a.o1 + (row * (a.K >> 8) + (s >> 3)) * 16);
    } else {
        r.l = ld_stream16(w + (row * nsub + s) * 16);
        r.h = ld_stream8(w + a.o1 + (row * nsub + s) * 8);
        r.sc = *reinterpret_cast<const uint16_t *>(w + a.o2 + row * (a.K >> 4) + 2 * s);
        r.d = *reinterpret_cast<const uint16_t *>(w + a.o3 + (row * (a.K >> 8) + (s >> 3)) * 2);
    }
}

// Unpacked weights of one row slot for one sub-block: eight dwords of int8
// codes in the activation's element order, plus the block's scale terms.
struct WDec {
    uint32_t v[8];
    float s0, s1;  // Q8_0: d; Q4_K: d*sc, dmin*m; Q6_K: d
    int32_t i0, i1;  // Q6_K: the two int8 sub-scales
};

template <int QT>
__device__ __forceinline__ void decode_w(WDec &o, const WRaw<QT> &r, int j8) {
    if constexpr (QT == SV_Q8_0) {
        o.v[0] = r.q0.x; o.v[1] = r.q0.y; o.v[2] = r.q0.z; o.v[3] = r.q0.w;
        o.v[4] = r.q1.x; o.v[5] = r.q1.y; o.v[6] = r.q1.z; o.v[7] = r.q1.w;
        o.s0 = half_bits_to_float(r.d);
    } else if constexpr (QT == SV_Q4_K) {
        const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            o.v[k] = q[k] & 0x0F0F0F0Fu;
            o.v[4 + k] = (q[k] >> 4) & 0x0F0F0F0Fu;
        }
        // 6-bit sub-scale and min of sub-block j8 from the packed 12 bytes
        // (header dwords y, z, w), see the Q4_K layout of ggml.
        const uint32_t sh = 8u * (j8 & 3);
        uint32_t sc, mn;
        if (j8 < 4) {
            sc = __builtin_amdgcn_ubfe(r.h.y, sh, 6);
            mn = __builtin_amdgcn_ubfe(r.h.z, sh, 6);
        } else {
            sc = __builtin_amdgcn_ubfe(r.h.w, sh, 4) | (__builtin_amdgcn_ubfe(r.h.y, sh + 6, 2) << 4);
            mn = __builtin_amdgcn_ubfe(r.h.w, sh + 4, 4) | (__builtin_amdgcn_ubfe(r.h.z, sh + 6, 2) << 4);
        }
        const float d = half_bits_to_float(r.h.x & 0xFFFFu);
        const float dmin = half_bits_to_float(r.h.x >> 16);
        o.s0 = d * static_cast<float>(sc);
        o.s1 = dmin * static_cast<float>(mn);
    } else {
        const uint32_t L[4] = {r.l.x, r.l.y, r.l.z, r.l.w};
        const uint32_t H[2] = {r.h.x, r.h.y};
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t nib = hh ? ((L[k] >> 4) & 0x0F0F0F0Fu) : (L[k] & 0x0F0F0F0Fu);
                uint32_t hb;
                if (k == 0) hb = H[hh] << 4;
                else if (k == 1) hb = H[hh] << 2;
                else if (k == 2) hb = H[hh];
                else hb = H[hh] >> 2;
                o.v[4 * hh + k] = nib | (hb & 0x30303030u);
            }
        }
        o.i0 = static_cast<int32_t>(static_cast<int8_t>(r.sc & 0xFFu));
        o.i1 = static_cast<int32_t>(static_cast<int8_t>(r.sc >> 8));
        o.s0 = half_bits_to_float(r.d);
    }
}

// Activation of one position for one sub-block, read from LDS.
struct ARec {
    uint32_t v[8];
    float d;
    float xf;       // Q4_K: fp32 sum of the 32 codes
    int32_t x0, x1; // Q6_K: -32 * (sum of codes of each 16-half)
};

// One block term for one (row slot, position), accumulated into acc.
template <int QT>
__device__ __forceinline__ float block_term(const WDec &w, const ARec &a, float acc) {
    int32_t S = 0;
    if constexpr (QT == SV_Q6_K) {
        int32_t S0 = 0, S1 = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) S0 = dot4(w.v[k], a.v[k], S0);
#pragma unroll
        for (int k = 4; k < 8; k++) S1 = dot4(w.v[k], a.v[k], S1);
        int32_t I = __mul24(w.i0, S0);
        I += __mul24(w.i1, S1);
        I += __mul24(w.i0, a.x0);
        I += __mul24(w.i1, a.x1);
        return fmaf(w.s0 * a.d, static_cast<float>(I), acc);
    } else {
#pragma unroll
        for (int k = 0; k < 8; k++) S = dot4(w.v[k], a.v[k], S);
        if constexpr (QT == SV_Q8_0) {
            return fmaf(w.s0 * a.d, static_cast<float>(S), acc);
        } else {
            const float inner = fmaf(-w.s1, a.xf, w.s0 * static_cast<float>(S));
            return fmaf(a.d, inner, acc);
        }
    }
}

__device__ __forceinline__ void read_act(ARec &r, const uint8_t *act_m, int CS, int sl) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(act_m + sl * 16);
    const uint4 hi = *reinterpret_cast<const uint4 *>(act_m + CS * 16 + sl * 16);
    r.v[0] = lo.x; r.v[1] = lo.y; r.v[2] = lo.z; r.v[3] = lo.w;
    r.v[4] = hi.x; r.v[5] = hi.y; r.v[6] = hi.z; r.v[7] = hi.w;
    r.d = reinterpret_cast<const float *>(act_m + CS * 32)[sl];
    const int2 x = reinterpret_cast<const int2 *>(act_m + CS * 36)[sl];
    r.x0 = x.x;
    r.x1 = x.y;
    r.xf = __int_as_float(x.x);
}

// Stage sub-blocks [s0, s0 + cs) of every position into LDS.
template <int QT, int M>
__device__ void stage_act(uint8_t *act, const MvArgs &a, int64_t s0, int cs, int CS) {
    const int64_t K = a.K, nsub = K >> 5;
    const int nhalf = M * cs * 2;
    for (int i = threadIdx.x; i < nhalf; i += kThreads) {
        const int m = i / (cs * 2), r = i % (cs * 2), sl = r >> 1, h = r & 1;
        const uint4 v = *reinterpret_cast<const uint4 *>(a.aq + m * K + (s0 + sl) * 32 + h * 16);
        *reinterpret_cast<uint4 *>(act + m * CS * kActRec + h * CS * 16 + sl * 16) = v;
    }
    for (int i = threadIdx.x; i < M * cs; i += kThreads) {
        const int m = i / cs, sl = i % cs;
        uint8_t *am = act + m * CS * kActRec;
        reinterpret_cast<float *>(am + CS * 32)[sl] = a.ad[m * nsub + s0 + sl];
        const int2 s = *reinterpret_cast<const int2 *>(a.as16 + m * (K >> 4) + 2 * (s0 + sl));
        int2 x;
        if constexpr (QT == SV_Q4_K) {
            x.x = __float_as_int(static_cast<float>(s.x + s.y));
            x.y = 0;
        } else {
            x.x = -32 * s.x;
            x.y = -32 * s.y;
        }
        reinterpret_cast<int2 *>(am + CS * 36)[sl] = x;
    }
}

template <int QT, int M, int GL>
__global__ __launch_bounds__(kThreads) void mv_kernel(MvArgs a) {
    constexpr int g = 1 << GL, G = 64 >> GL;
    constexpr int ROWS = 4 * G * kR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> GL, jl = lane & (g - 1);
    const int j8 = jl & 7;
    const int64_t nsub = a.K >> 5;
    const int CS = a.chunk_sub;
    const int nchunks = static_cast<int>((nsub + CS - 1) / CS);

    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t *act = smem;
    float *ystage = reinterpret_cast<float *>(smem + M * CS * kActRec);
    float *rscale = ystage + a.n_w * M * ROWS;
    unsigned long long *bestbuf = reinterpret_cast<unsigned long long *>(rscale + SV_MAX_M);

    // RMS factor of the input (fixed order: lane-strided sequential sums,
    // then a butterfly over the wave).
    for (int m = wave; m < M; m += 4) {
        float r = 1.0f;
        if (a.in_parts) {
            float s = 0.0f;
            for (int i = lane; i < a.n_parts; i += 64) s += a.in_parts[m * a.n_parts + i];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
            r = 1.0f / sqrtf(s / static_cast<float>(a.K) + a.eps);
        }
        if (lane == 0) rscale[m] = r;
    }

    unsigned long long best[M];
#pragma unroll
    for (int m = 0; m < M; m++) best[m] = 0ull;

    bool staged_once = false;
    for (int tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
        const int64_t row0 = static_cast<int64_t>(tile) * ROWS;
        const int slot0 = (wave * G + grp) * kR;
        for (int mat = 0; mat < a.n_w; mat++) {
            const uint8_t *__restrict__ w = a.w[mat];
            int64_t srow[kR];
#pragma unroll
            for (int p = 0; p < kR; p++) {
                int64_t rr = row0 + slot0 + p;
                if (rr >= a.N) rr = 0;
                int64_t sr = a.row_ids ? static_cast<int64_t>(a.row_ids[rr]) : rr;
                // Out-of-range ids are a caller error; clamp so no read
                // leaves the matrix.
                srow[p] = (sr < 0 || sr >= a.wrows) ? 0 : sr;
            }
            float acc[kR][M];
#pragma unroll
            for (int p = 0; p < kR; p++)
#pragma unroll
                for (int m = 0; m < M; m++) acc[p][m] = 0.0f;

            for (int c = 0; c < nchunks; c++) {
                const int64_t s0 = static_cast<int64_t>(c) * CS;
                const int cs = static_cast<int>(std::min<int64_t>(CS, nsub - s0));
                if (nchunks > 1 || !staged_once) {
                    __syncthreads();
                    stage_act<QT, M>(act, a, s0, cs, CS);
                    __syncthreads();
                    staged_once = true;
                }
                const int T = (cs + g - 1) / g;
                WRaw<QT> raw[kR];
                if (jl < cs) {
#pragma unroll
                    for (int p = 0; p < kR; p++) load_w<QT>(raw[p], w, a, srow[p], s0 + jl);
                }
                for (int t = 0; t < T; t++) {
                    const int sl = jl + g * t;
                    const bool valid = sl < cs;
                    WDec dec[kR];
                    if (valid) {
#pragma unroll
                        for (int p = 0; p < kR; p++) decode_w<QT>(dec[p], raw[p], j8);
                    }
                    if (sl + g < cs) {
#pragma unroll
                        for (int p = 0; p < kR; p++) load_w<QT>(raw[p], w, a, srow[p], s0 + sl + g);
                    }
                    if (valid) {
#pragma unroll
                        for (int m = 0; m < M; m++) {
                            ARec ar;
                            read_act(ar, act + m * CS * kActRec, CS, sl);
#pragma unroll
                            for (int p = 0; p < kR; p++) acc[p][m] = block_term<QT>(dec[p], ar, acc[p][m]);
                        }
                    }
                }
            }
            // Combine the g lanes of each group (butterfly; all lanes end
            // with the same value) and stage the scaled result.
#pragma unroll
            for (int p = 0; p < kR; p++)
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float v = acc[p][m];
#pragma unroll
                    for (int o = g >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
                    acc[p][m] = v;
                }
            if (jl == 0) {
#pragma unroll
                for (int p = 0; p < kR; p++)
#pragma unroll
                    for (int m = 0; m < M; m++) ystage[(mat * M + m) * ROWS + slot0 + p] = acc[p][m] * rscale[m];
            }
        }
        __syncthreads();
        const int rows_here = static_cast<int>(std::min<int64_t>(ROWS, a.N - row0));
        // Outputs, coalesced.
        for (int mat = 0; mat < a.n_w; mat++) {
            if (!a.y[mat]) continue;
            for (int i = threadIdx.x; i < M * ROWS; i += kThreads) {
                const int m = i / ROWS, r = i % ROWS;
                if (r < rows_here) a.y[mat][m * a.N + row0 + r] = ystage[(mat * M + m) * ROWS + r];
            }
        }
        // Fused argmax over this tile's rows.
        if (a.argmax) {
            for (int m = 0; m < M; m++) {
                unsigned long long b = 0ull;
                for (int r = threadIdx.x; r < rows_here; r += kThreads)
                        b = umax64(b, pack_argmax(ystage[m * ROWS + r], static_cast<uint32_t>(row0 + r)));
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) b = umax64(b, __shfl_xor(b, o, 64));
                best[m] = umax64(best[m], b);
            }
        }
        // Fused requantisation for the next consumer.
        if (a.ep_mode != SV_EP_NONE) {
            const int nblk = rows_here / 32;
            const int hw = threadIdx.x >> 5, l32 = threadIdx.x & 31;
            for (int it = hw; it < M * nblk; it += kThreads / 32) {
                const int m = it / nblk, blk = it % nblk;
                const int r = blk * 32 + l32;
                float v;
                if (a.ep_mode == SV_EP_PAIR) v = ystage[(0 * M + m) * ROWS + r] * ystage[(1 * M + m) * ROWS + r];
                else v = ystage[(a.ep_src * M + m) * ROWS + r];
                const int64_t grow = row0 + r;
                const float vg = a.gamma ? v * a.gamma[grow] : v;
                float am = fabsf(vg);
#pragma unroll
                for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 32));
                const float dd = am / 127.0f;
                const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
                float rq = roundf(vg * id);
                rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                const int qi = static_cast<int>(rq);
                a.oq[m * a.N + grow] = static_cast<int8_t>(qi);
                int s = qi;
#pragma unroll
                for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 32);
                float sq = v * v;
#pragma unroll
                for (int o = 16; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 32);
                const int64_t gb = grow >> 5;
                if ((l32 & 15) == 0) a.os16[m * (a.N >> 4) + 2 * gb + (l32 >> 4)] = s;
                if (l32 == 0) {
                    a.od[m * (a.N >> 5) + gb] = dd;
                    a.osumsq[m * (a.N >> 5) + gb] = sq;
                }
            }
        }
        __syncthreads();
    }
    if (a.argmax) {
        for (int m = 0; m < M; m++) {
            if (lane == 0) bestbuf[wave * SV_MAX_M + m] = best[m];
        }
        __syncthreads();
        if (threadIdx.x < M) {
            unsigned long long b = 0ull;
            for (int wv = 0; wv < 4; wv++) b = umax64(b, bestbuf[wv * SV_MAX_M + threadIdx.x]);
            if (b) atomicMax(a.argmax + threadIdx.x, b);
        }
    }
}

__global__ void zero_u64(unsigned long long *p, int n) {
    if (static_cast<int>(threadIdx.x) < n) p[threadIdx.x] = 0ull;
}

// ------------------------------------------------------------- dispatch
using KernelFn = void (*)(MvArgs);

template <int QT, int GL, int M>
static KernelFn pick_m(int m) {
    if constexpr (M > SV_MAX_M) {
        return nullptr;
    } else {
        if (m == M) return mv_kernel<QT, M, GL>;
        return pick_m<QT, GL, M + 1>(m);
    }
}

template <int QT>
static KernelFn pick(int gl, int m) {
    if (gl == 5) return pick_m<QT, 5, 1>(m);
    return pick_m<QT, 4, 1>(m);
}

static KernelFn pick_kernel(int qt, int gl, int m) {
    if (qt == SV_Q8_0) return pick<SV_Q8_0>(gl, m);
    if (qt == SV_Q4_K) return pick<SV_Q4_K>(gl, m);
    return pick<SV_Q6_K>(gl, m);
}

// Lanes per row group: 32 when the sub-block count allows a full-width
// split, else 16.  A function of K only.
static int group_log2(int64_t K) {
    const int64_t nsub = K / 32;
    return (nsub % 32 == 0) ? 5 : 4;
}

static int validate_act(const sv_act *A) {
    SV_REQUIRE(A, SV_ERR_ARG, "activation descriptor is NULL");
    SV_REQUIRE(A->M >= 1 && A->M <= SV_MAX_M, SV_ERR_ARG, "M must be in [1, 16]");
    SV_REQUIRE(A->q && A->d && A->s16, SV_ERR_ARG, "activation buffers must not be NULL");
    SV_REQUIRE(A->K > 0 && A->K % 32 == 0, SV_ERR_SHAPE, "activation K must be a positive multiple of 32");
    SV_REQUIRE(aligned(A->q, 16) && aligned(A->d, 4) && aligned(A->s16, 8), SV_ERR_ALIGN,
               "activation codes must be 16-byte aligned, scales 4-byte, sums 8-byte");
    if (A->sumsq_parts) {
        SV_REQUIRE(A->n_parts >= 1, SV_ERR_ARG, "n_parts must be >= 1 when sumsq_parts is given");
        SV_REQUIRE(aligned(A->sumsq_parts, 4), SV_ERR_ALIGN, "sumsq_parts must be 4-byte aligned");
    }
    return SV_OK;
}

static int validate_weight(const sv_weight &W, int64_t K) {
    SV_REQUIRE(W.data, SV_ERR_ARG, "weight data is NULL");
    SV_REQUIRE(W.qtype == SV_Q8_0 || W.qtype == SV_Q4_K || W.qtype == SV_Q6_K, SV_ERR_QTYPE,
               "unsupported qtype " + std::to_string(W.qtype));
    Streams s;
    SV_REQUIRE(streams_of(W.qtype, W.rows, W.cols, &s), SV_ERR_SHAPE,
               "weight cols must be a multiple of 32 (Q8_0) or 256 (Q4_K, Q6_K)");
    SV_REQUIRE(W.cols == K, SV_ERR_SHAPE, "weight cols must equal the activation K");
    SV_REQUIRE(W.rows < (1ll << 31), SV_ERR_SHAPE, "weight rows must be < 2^31");
    SV_REQUIRE(aligned(W.data, 256), SV_ERR_ALIGN, "repacked weights must be 256-byte aligned");
    return SV_OK;
}

static int launch(MvArgs &a, int qt, int M, int grid_cap, hipStream_t st) {
    const int gl = group_log2(a.K);
    const int g = 1 << gl;
    const int rows_tile = 4 * (64 >> gl) * kR;
    const int64_t nsub = a.K / 32;
    const int fixed = a.n_w * M * rows_tile * 4 + SV_MAX_M * 4 + 4 * SV_MAX_M * 8;
    int cs = static_cast<int>((kLdsBudget - fixed) / (M * kActRec));
    cs = (cs / g) * g;
    const int64_t nsub_r = (nsub + g - 1) / g * g;
    if (cs > nsub_r) cs = static_cast<int>(nsub_r);
    SV_REQUIRE(cs >= g, SV_ERR_SHAPE, "internal: LDS chunk too small");
    a.chunk_sub = cs;
    const int64_t tiles = (a.N + rows_tile - 1) / rows_tile;
    SV_REQUIRE(tiles < (1ll << 31), SV_ERR_SHAPE, "too many rows");
    a.n_tiles = static_cast<int>(tiles);
    const int grid = static_cast<int>(std::min<int64_t>(tiles, grid_cap));
    const size_t lds = static_cast<size_t>(M) * cs * kActRec + fixed;
    KernelFn fn = pick_kernel(qt, gl, M);
    SV_REQUIRE(fn, SV_ERR_ARG, "internal: no kernel for this M");
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, st, a);
    return hip_check(hipGetLastError(), "verify_matvec launch");
}

static void fill_act(MvArgs &a, const sv_act *A) {
    a.K = A->K;
    a.aq = A->q;
    a.ad = A->d;
    a.as16 = A->s16;
    a.in_parts = A->sumsq_parts;
    a.n_parts = A->sumsq_parts ? A->n_parts : 0;
    a.eps = A->eps;
}

}  // namespace sv

extern "C" int sv_verify_matvec(const sv_weight *W, int32_t n_w, const sv_act *A, float *const *y,
                                const sv_epilogue *ep, void *stream) {
    using namespace sv;
    SV_REQUIRE(W, SV_ERR_ARG, "verify_matvec: W is NULL");
    SV_REQUIRE(n_w >= 1 && n_w <= 3, SV_ERR_ARG, "verify_matvec: n_w must be 1..3");
    int rc = validate_act(A);
    if (rc) return rc;
    for (int i = 0; i < n_w; i++) {
        rc = validate_weight(W[i], A->K);
        if (rc) return rc;
        SV_REQUIRE(W[i].qtype == W[0].qtype && W[i].rows == W[0].rows, SV_ERR_SHAPE,
                   "verify_matvec: matrices sharing an input must have the same qtype and rows");
    }
    MvArgs a{};
    a.n_w = n_w;
    a.N = W[0].rows;
    a.wrows = W[0].rows;
    Streams s;
    streams_of(W[0].qtype, W[0].rows, W[0].cols, &s);
    a.o1 = s.off[1];
    a.o2 = s.off[2];
    a.o3 = s.off[3];
    for (int i = 0; i < n_w; i++) {
        a.w[i] = static_cast<const uint8_t *>(W[i].data);
        a.y[i] = y ? y[i] : nullptr;
        if (a.y[i]) SV_REQUIRE(aligned(a.y[i], 4), SV_ERR_ALIGN, "verify_matvec: y must be 4-byte aligned");
    }
    fill_act(a, A);
    a.ep_mode = SV_EP_NONE;
    if (ep && ep->mode != SV_EP_NONE) {
        SV_REQUIRE(ep->mode == SV_EP_QUANT || ep->mode == SV_EP_PAIR, SV_ERR_ARG, "verify_matvec: bad epilogue mode");
        SV_REQUIRE(a.N % 32 == 0, SV_ERR_SHAPE, "verify_matvec: epilogue needs rows % 32 == 0");
        SV_REQUIRE(ep->q && ep->d && ep->s16 && ep->sumsq, SV_ERR_ARG, "verify_matvec: epilogue outputs are NULL");
        SV_REQUIRE(aligned(ep->q, 16) && aligned(ep->d, 4) && aligned(ep->s16, 8) && aligned(ep->sumsq, 4) &&
                       (!ep->gamma || aligned(ep->gamma, 4)),
                   SV_ERR_ALIGN, "verify_matvec: epilogue buffer alignment");
        if (ep->mode == SV_EP_QUANT)
            SV_REQUIRE(ep->src >= 0 && ep->src < n_w, SV_ERR_ARG, "verify_matvec: epilogue src out of range");
        else
            SV_REQUIRE(n_w == 2, SV_ERR_ARG, "verify_matvec: pair epilogue needs exactly two matrices");
        a.ep_mode = ep->mode;
        a.ep_src = ep->src;
        a.gamma = ep->gamma;
        a.oq = ep->q;
        a.od = ep->d;
        a.os16 = ep->s16;
        a.osumsq = ep->sumsq;
    }
    return launch(a, W[0].qtype, A->M, 1 << 30, as_stream(stream));
}

extern "C" int sv_head_logits(const sv_weight *H, const sv_act *A, const int32_t *row_ids, int64_t n_rows,
                              float *logits, uint64_t *argmax, void *stream) {
    using namespace sv;
    SV_REQUIRE(H, SV_ERR_ARG, "head_logits: H is NULL");
    int rc = validate_act(A);
    if (rc) return rc;
    rc = validate_weight(*H, A->K);
    if (rc) return rc;
    if (!row_ids) n_rows = H->rows;
    SV_REQUIRE(n_rows >= 1 && n_rows < (1ll << 31), SV_ERR_SHAPE, "head_logits: n_rows out of range");
    SV_REQUIRE(logits || argmax, SV_ERR_ARG, "head_logits: nothing to write");
    SV_REQUIRE(!logits || aligned(logits, 4), SV_ERR_ALIGN, "head_logits: logits must be 4-byte aligned");
    SV_REQUIRE(!argmax || aligned(argmax, 8), SV_ERR_ALIGN, "head_logits: argmax must be 8-byte aligned");
    SV_REQUIRE(!row_ids || aligned(row_ids, 4), SV_ERR_ALIGN, "head_logits: row_ids must be 4-byte aligned");
    MvArgs a{};
    a.n_w = 1;
    a.N = n_rows;
    a.wrows = H->rows;
    Streams s;
    streams_of(H->qtype, H->rows, H->cols, &s);
    a.o1 = s.off[1];
    a.o2 = s.off[2];
    a.o3 = s.off[3];
    a.w[0] = static_cast<const uint8_t *>(H->data);
    a.y[0] = logits;
    a.row_ids = row_ids;
    a.argmax = reinterpret_cast<unsigned long long *>(argmax);
    fill_act(a, A);
    a.ep_mode = SV_EP_NONE;
    hipStream_t st = as_stream(stream);
    if (argmax) {
        hipLaunchKernelGGL(zero_u64, dim3(1), dim3(64), 0, st, a.argmax, A->M);
        rc = hip_check(hipGetLastError(), "head_logits init");
        if (rc) return rc;
    }
    return launch(a, H->qtype, A->M, 1024, st);
}
