// matvec_dev.h - device code of the verification projection (a3), its
// fused producer epilogue (a4), the output head with fused argmax (a6, a9)
// and the phase sequencing of a whole pass in one persistent launch (a5).
// Included by matvec_inst.hip only, which instantiates the kernels for one M.
//
// One weight stream serves all M positions ("Inside OpenJet Engine: making
// speculative decoding pay", section "One GPU launch for a speculative
// cycle": weight reads serve multiple verification positions, activation
// loads are reused across weight rows, and one launch carries the phases of
// a cycle separated by grid-wide synchronisation).
//
// Work decomposition.  A phase (one to three matrices sharing an input) is
// cut into units = (32-row tile, K chunk, matrix):
//  * K is walked in steps of 256 elements (one K-quant super-block, eight
//    Q8_0 blocks); a chunk is at most 12 steps, so S(K) = ceil(steps / 12)
//    depends on K alone.  Wave w takes the 16-row half tile w & 1 over the
//    half w >> 1 of the chunk's steps, so all four waves carry the same
//    rows x steps.
//  * Lane j of an 8-lane row group reads sub-block 8t + j of two rows: the
//    group reads 128 contiguous bytes of a row, and each weight record is
//    read once and reused from registers for all M positions.  The input
//    chunk is staged in LDS once per unit.
// Arithmetic.  Integer block sums come from v_dot4 (exact); each block's
// fp32 combine is a fixed sequence of operations per (row, position); a lane
// adds its blocks in increasing order, the 8 lanes of a group are combined
// in a fixed DPP tree, the step parts in order and the K chunks in chunk
// order.  Nothing depends on M or on which workgroup ran which unit,
// so every output row is bit-identical to the same row computed alone, and
// runs are deterministic.
// Scheduling.  Single calls launch one workgroup per unit.  A whole pass
// runs as one persistent launch sized to the number of workgroups the GPU
// holds at once: the units of each phase are dealt round-robin, and a
// workgroup issues a unit's weight loads before it waits until the phase its
// input comes from has handed off.  All waits are bounded.
#pragma once
#include <algorithm>
#include <vector>

#include "matvec_launch.h"

namespace sv {


// Lane layout of a unit: R rows per lane; the tile's rows are cut into
// RS = 4 / R parts and the chunk's steps into SS = 4 / RS parts, wave w
// taking row part w % RS over step part w / RS (at most WS steps).  Two rows
// per lane give every wave the same rows x steps (a chunk's step count is
// rarely a multiple of four).  The layout fixes the order of the fp32 sums,
// so it must not depend on M: each position's result is bitwise the same at
// every M.
struct Lay {
    static constexpr int R = 2;
    static constexpr int RS = 4 / R;
    static constexpr int SS = 4 / RS;
    static constexpr int WS = kMaxChunkSteps / SS;
};


// ------------------------------------------------------------ weights
template <int QT>
struct WRaw;
template <>
struct WRaw<SV_Q8_0> {
    uint4 q0, q1;
    uint32_t d;
};
// The Q4_K super-block header (16 bytes per row and step) is spread over a
// quad of lanes, one dword each, and shared at decode time with quad
// permutes instead of every lane holding a copy.
template <>
struct WRaw<SV_Q4_K> {
    uint4 q;
    uint32_t h;   // header dword (lane & 3): d|dmin, scale/min bytes 0-3, 4-7, 8-11
};
template <>
struct WRaw<SV_Q6_K> {
    uint4 l;
    uint2 h;
    uint32_t sc, d;
};

template <int QT>
__device__ __forceinline__ void load_w(WRaw<QT> &r, const uint8_t *__restrict__ w, const PhaseDesc &P, int64_t row,
                                       int64_t s) {
    const int64_t K = P.K, nsub = K >> 5;
    if constexpr (QT == SV_Q8_0) {
        r.q0 = gld16_nt(w + row * K + s * 32);
        r.q1 = gld16_nt(w + row * K + s * 32 + 16);
        r.d = gld(reinterpret_cast<const uint16_t *>(w + P.o1 + (row * nsub + s) * 2));
    } else if constexpr (QT == SV_Q4_K) {
        r.q = gld16_nt(w + (row * nsub + s) * 16);
        r.h = gld(reinterpret_cast<const uint32_t *>(w + P.o1 + (row * (K >> 8) + (s >> 3)) * 16) + (s & 3));
    } else {
        r.l = gld16_nt(w + (row * nsub + s) * 16);
        r.h = gld8_nt(w + P.o1 + (row * nsub + s) * 8);
        r.sc = gld(reinterpret_cast<const uint16_t *>(w + P.o2 + row * (K >> 4) + 2 * s));
        r.d = gld(reinterpret_cast<const uint16_t *>(w + P.o3 + (row * (K >> 8) + (s >> 3)) * 2));
    }
}

// Unpacked weights of one row slot for one sub-block: eight dwords of int8
// codes in the activation's element order, plus the block's scale terms.
struct WDec {
    uint32_t v[8];
    float s0, s1;    // Q8_0: d; Q4_K: d*sc, dmin*m; Q6_K: d
    int32_t i0, i1;  // Q6_K: the two int8 sub-scales
};

// Value of quad lane i (CTRL = i * 0x55) of v in every lane of each quad.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

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
        // 6-bit sub-scale and min of sub-block j8 from the 12 packed bytes
        // (header dwords y, z, w) of the ggml Q4_K layout.
        const uint32_t hx = quad_bcast<0x00>(r.h), hy = quad_bcast<0x55>(r.h);
        const uint32_t hz = quad_bcast<0xAA>(r.h), hw = quad_bcast<0xFF>(r.h);
        const uint32_t sh = 8u * (j8 & 3);
        uint32_t sc, mn;
        if (j8 < 4) {
            sc = __builtin_amdgcn_ubfe(hy, sh, 6);
            mn = __builtin_amdgcn_ubfe(hz, sh, 6);
        } else {
            sc = __builtin_amdgcn_ubfe(hw, sh, 4) | (__builtin_amdgcn_ubfe(hy, sh + 6, 2) << 4);
            mn = __builtin_amdgcn_ubfe(hw, sh + 4, 4) | (__builtin_amdgcn_ubfe(hz, sh + 6, 2) << 4);
        }
        const float d = half_bits_to_float(hx & 0xFFFFu);
        const float dmin = half_bits_to_float(hx >> 16);
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
    int32_t x0, x1;  // exact sums of the codes of each 16-element half
};

// Per-position terms of a sub-block shared by the row slots of a lane:
// Q4_K's fp32 code sum (min term), Q6_K's -32 offset of each half as the
// starting value of that half's integer dot product.
struct AExt {
    float xf;
    int32_t o0, o1;
};
template <int QT>
__device__ __forceinline__ AExt act_ext(const ARec &a) {
    AExt e;
    e.xf = static_cast<float>(a.x0 + a.x1);
    e.o0 = -32 * a.x0;
    e.o1 = -32 * a.x1;
    return e;
}

// One block term for one (row slot, position), accumulated into acc.  All
// integer parts are exact, so the value does not depend on how they are
// grouped: Q6_K's sum over (q - 32) a of each half is the dot product of the
// stored 6-bit codes started at -32 * (sum of a).
template <int QT>
__device__ __forceinline__ float block_term(const WDec &w, const ARec &a, const AExt &e, float acc) {
    if constexpr (QT == SV_Q6_K) {
        int32_t S0 = dot4_from(w.v[0], a.v[0], e.o0), S1 = dot4_from(w.v[4], a.v[4], e.o1);
#pragma unroll
        for (int k = 1; k < 4; k++) S0 = dot4(w.v[k], a.v[k], S0);
#pragma unroll
        for (int k = 5; k < 8; k++) S1 = dot4(w.v[k], a.v[k], S1);
        const int32_t I = __mul24(w.i0, S0) + __mul24(w.i1, S1);
        return fmaf(w.s0 * a.d, static_cast<float>(I), acc);
    } else {
        int32_t S = dot4_first(w.v[0], a.v[0]);
#pragma unroll
        for (int k = 1; k < 8; k++) S = dot4(w.v[k], a.v[k], S);
        if constexpr (QT == SV_Q8_0) {
            return fmaf(w.s0 * a.d, static_cast<float>(S), acc);
        } else {
            const float inner = fmaf(-w.s1, e.xf, w.s0 * static_cast<float>(S));
            return fmaf(a.d, inner, acc);
        }
    }
}

// LDS record of the staged activation chunk, per position: [CS] 16-byte low
// halves, [CS] 16-byte high halves, [CS] fp32 scales, [CS] 8-byte sums.
__device__ __forceinline__ void read_act(ARec &r, const uint8_t *act_m, int CS, int sl) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(act_m + sl * 16);
    const uint4 hi = *reinterpret_cast<const uint4 *>(act_m + CS * 16 + sl * 16);
    r.v[0] = lo.x; r.v[1] = lo.y; r.v[2] = lo.z; r.v[3] = lo.w;
    r.v[4] = hi.x; r.v[5] = hi.y; r.v[6] = hi.z; r.v[7] = hi.w;
    r.d = reinterpret_cast<const float *>(act_m + CS * 32)[sl];
    const int2 x = reinterpret_cast<const int2 *>(act_m + CS * 36)[sl];
    r.x0 = x.x;
    r.x1 = x.y;
}

// Shared state of a workgroup.
template <int M>
struct Shared {
    float rscale[SV_MAX_M];
    unsigned long long best[SV_MAX_M];
    int last;
    unsigned abort;
    unsigned long long t_wait, t_staged, t_computed, t_reduced, t_epi;   // first unit of a phase (trace)
};

// Workgroup barrier for LDS data only: waits for this wave's LDS
// operations, not for its outstanding global loads (a full __syncthreads
// would also wait for weight records already requested for the next unit).
// No global memory written before it is read by another wave after it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


__device__ __forceinline__ bool wait_ready(const unsigned *ctr, unsigned target, unsigned *status, unsigned &abort_sh) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        unsigned n = 0;
        bool ok = true;
        // two polls in flight: the next read is issued before the previous
        // one is examined, so an update is seen about half a round trip
        // sooner than with one read at a time
        // every lane reads (lanes >= kSlots repeat the first slots), so no
        // branch hides the loads from the wait-count bookkeeping
        const int rep = static_cast<int>(blockIdx.x % kReplicas);
        const unsigned *slot = ctr + (rep * kSlots + (lane & (kSlots - 1))) * kSlotStride;
        unsigned a = ld_dev(slot);
        for (;;) {
            __builtin_amdgcn_s_sleep(2);
            const unsigned b = ld_dev(slot);
            unsigned v = (lane < kSlots) ? a : 0u;
#pragma unroll
            for (int o = 4; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
            v = __shfl(v, 0, 64);
            if (v >= target) break;
            if (++n > kSpinLimit || ((n & 63u) == 0u && ld_dev(status) != 0u)) {
                ok = false;
                break;
            }
            a = b;
        }
        if (lane == 0) {
            if (!ok) or_dev(status, 1u);
            abort_sh = ok ? 0u : 1u;
        }
    }
    __syncthreads();
    return abort_sh == 0u;
}


// Stage positions [m0, m0 + mg) of the chunk's sub-blocks [s0, s0 + cs) into
// LDS.  Thread t takes items t, t + 256, ... of the 16-byte halves and of the
// (scale, sums) records; every global load of a thread is issued before the
// first one is stored.  The item index i splits into (position, offset) as
// i / D = (i * ceil(2^20 / D)) >> 20, exact for i < 2^11 and D <= 512 (the
// rounding error i / 2^20 stays below 1 / D), so no lane divides.
constexpr int kStageHalf = 6;   // >= 8 positions * 96 sub-blocks * 2 halves / 256 threads
constexpr int kStageRec = 3;    // >= 8 * 96 / 256

__device__ __forceinline__ void stage_act(uint8_t *act, const PhaseDesc &P, int m0, int mg, int64_t s0, int cs,
                                          int CS) {
    const int64_t K = P.K, nsub = K >> 5;
    const int nhalf = mg * cs * 2, nrec = mg * cs;
    const uint32_t D2 = 2u * static_cast<uint32_t>(cs), D1 = static_cast<uint32_t>(cs);
    const uint32_t mul2 = ((1u << 20) + D2 - 1) / D2, mul1 = ((1u << 20) + D1 - 1) / D1;
    // named registers, not arrays: a private array here ends up in scratch
    uint4 h0, h1, h2, h3, h4, h5;
#define SV_HALF(k)                                                                                       \
    const int i = threadIdx.x + (k) * kThreads;                                                          \
    const int m = static_cast<int>(__umul24(static_cast<uint32_t>(i), mul2) >> 20);                      \
    const int r = i - m * static_cast<int>(D2), sl = r >> 1, h = r & 1;
#define SV_LDH(k, hv)                                                                                    \
    {                                                                                                    \
        SV_HALF(k)                                                                                       \
        if (i < nhalf) hv = gld16(P.aq + (m0 + m) * K + (s0 + sl) * 32 + h * 16);                         \
    }
    SV_LDH(0, h0) SV_LDH(1, h1) SV_LDH(2, h2) SV_LDH(3, h3) SV_LDH(4, h4) SV_LDH(5, h5)
#undef SV_LDH
    float d0, d1, d2;
    uint2 x0, x1, x2;
#define SV_REC(k)                                                                                        \
    const int i = threadIdx.x + (k) * kThreads;                                                          \
    const int m = static_cast<int>(__umul24(static_cast<uint32_t>(i), mul1) >> 20);                      \
    const int sl = i - m * static_cast<int>(D1);
#define SV_LDR(k, dv, xv)                                                                                \
    {                                                                                                    \
        SV_REC(k)                                                                                        \
        if (i < nrec) {                                                                                  \
            dv = gld(P.ad + (m0 + m) * nsub + s0 + sl);                                                  \
            xv = gld8(P.as16 + (m0 + m) * (K >> 4) + 2 * (s0 + sl));                                     \
        }                                                                                                \
    }
    SV_LDR(0, d0, x0) SV_LDR(1, d1, x1) SV_LDR(2, d2, x2)
#undef SV_LDR
#define SV_STH(k, hv)                                                                                    \
    {                                                                                                    \
        SV_HALF(k)                                                                                       \
        if (i < nhalf) *reinterpret_cast<uint4 *>(act + m * CS * kActRec + h * CS * 16 + sl * 16) = hv;    \
    }
    SV_STH(0, h0) SV_STH(1, h1) SV_STH(2, h2) SV_STH(3, h3) SV_STH(4, h4) SV_STH(5, h5)
#undef SV_STH
#define SV_STR(k, dv, xv)                                                                                \
    {                                                                                                    \
        SV_REC(k)                                                                                        \
        if (i < nrec) {                                                                                  \
            uint8_t *am = act + m * CS * kActRec;                                                        \
            reinterpret_cast<float *>(am + CS * 32)[sl] = dv;                                            \
            reinterpret_cast<uint2 *>(am + CS * 36)[sl] = xv;                                            \
        }                                                                                                \
    }
    SV_STR(0, d0, x0) SV_STR(1, d1, x1) SV_STR(2, d2, x2)
#undef SV_STR
#undef SV_HALF
#undef SV_REC
}

// Sums over lanes with data-parallel primitives (no LDS traffic), in a fixed
// order.  DPP controls: quad_perm, row_shl:n = 0x100 + n, row_ror:n = 0x120 + n.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7)) of each group of eight
// lanes, in the group's lane 0.
__device__ __forceinline__ float group8_sum(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x104>(v);   // row_shl:4
    return v;
}
// Sum of the 64 lanes of the wave (every lane gets it): quads, then rows
// of 16, then the four rows in order.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x124>(v);   // row_ror:4
    v += dpp_f<0x128>(v);   // row_ror:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((r0 + r1) + r2) + r3;
}

// RMS factors r = 1 / sqrt(sum / K + eps) of the input rows from its
// per-block sums of squares.  rms_fetch copies the M x n_parts partials into
// LDS with the loads' LDS transfer (no registers held), issued with the
// input staging; after the barrier that ends staging, rms_store has wave w
// take positions w + 4 k: lane l adds partials l, l + 64, ... in order, then
// wave_sum.  A fixed order that depends only on the number of partials.
__device__ __forceinline__ void rms_fetch(float *parts, const PhaseDesc &P, int M) {
    const int lane = threadIdx.x & 63;
    const int wave = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    const int total = M * P.n_parts;
    for (int k = wave; 64 * k < total; k += 4) {
        const int f = 64 * k + lane;
        if (f < total)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(P.in_parts + f),
                                             (__attribute__((address_space(3))) void *)(parts + 64 * k), 4, 0, 0);
    }
}

__device__ __forceinline__ void rms_store(const float *parts, const PhaseDesc &P, int M, float *rs) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int m = wave; m < M; m += 4) {
        float t = 0.0f;
        for (int i = lane; i < P.n_parts; i += 64) t += parts[m * P.n_parts + i];
        const float tot = wave_sum(t);
        if (lane == 0) rs[m] = 1.0f / sqrtf(tot / static_cast<float>(P.K) + P.eps);
    }
}

// Reductions over the 32 lanes of a half-wave (every lane gets the result):
// within each row of 16 by DPP, then the two rows by one lane exchange.
__device__ __forceinline__ float half_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x128>(v));
    return fmaxf(v, __shfl_xor(v, 16, 64));
}
__device__ __forceinline__ float half_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x128>(v);
    return v + __shfl_xor(v, 16, 64);
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
// integer sum over each row of 16 lanes
__device__ __forceinline__ int row_sum(int v) {
    v += dpp_i<0xB1>(v);
    v += dpp_i<0x4E>(v);
    v += dpp_i<0x124>(v);
    v += dpp_i<0x128>(v);
    return v;
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const int lo = dpp_i<CTRL>(static_cast<int>(v & 0xFFFFFFFFull));
    const int hi = dpp_i<CTRL>(static_cast<int>(v >> 32));
    return (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}
__device__ __forceinline__ unsigned long long half_max64(unsigned long long v) {
    v = umax64(v, dpp_u64<0xB1>(v));
    v = umax64(v, dpp_u64<0x4E>(v));
    v = umax64(v, dpp_u64<0x124>(v));
    v = umax64(v, dpp_u64<0x128>(v));
    return umax64(v, __shfl_xor(v, 16, 64));
}

// Epilogue of a finished row tile (LDS ystage [n_w][M][kRows]): y outputs
// of the matrices in [mat_lo, mat_hi), argmax candidates and the requantised
// next activation.  Half-wave h takes positions h, h + 8 (lane = row).
template <int M>
__device__ __forceinline__ void finish_tile(const PhaseDesc &P, const float *ystage, int64_t row0, int mat_lo,
                                            int mat_hi, bool do_ep, float g_row, Shared<M> &sh) {
    const int rows_here = static_cast<int>(min(static_cast<int64_t>(kRows), static_cast<int64_t>(P.N) - row0));
    for (int mat = mat_lo; mat < mat_hi; mat++) {
        float *y = P.y[mat];
        if (!y) continue;
        for (int i = threadIdx.x; i < M * kRows; i += kThreads) {
            const int m = i / kRows, r = i % kRows;
            if (r < rows_here) gst(y + static_cast<int64_t>(m) * P.N + row0 + r, ystage[(mat * M + m) * kRows + r]);
        }
    }
    const int hw = threadIdx.x >> 5, l32 = threadIdx.x & 31;
    if (P.argmax) {
        for (int m = hw; m < M; m += kThreads / 32) {
            const unsigned long long key =
                l32 < rows_here ? pack_argmax(ystage[m * kRows + l32], static_cast<uint32_t>(row0 + l32)) : 0ull;
            const unsigned long long b = half_max64(key);
            if (l32 == 0 && b) atomicMax(&sh.best[m], b);
        }
    }
    if (do_ep && P.ep_mode != SV_EP_NONE && rows_here == kRows) {
        const int64_t N = P.N;
        for (int m = hw; m < M; m += kThreads / 32) {
            float v;
            if (P.ep_mode == SV_EP_PAIR) v = ystage[(0 * M + m) * kRows + l32] * ystage[(1 * M + m) * kRows + l32];
            else v = ystage[(P.ep_src * M + m) * kRows + l32];
            const int64_t grow = row0 + l32;
            const float vg = P.gamma ? v * g_row : v;
            const float am = half_max(fabsf(vg));
            const float dd = am / 127.0f;
            const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
            float rq = roundf(vg * id);
            rq = fminf(fmaxf(rq, -127.0f), 127.0f);
            const int qi = static_cast<int>(rq);
            const int s = row_sum(qi);
            const float sq = half_sum(v * v);
            st_dev(P.oq + m * N + grow, static_cast<int8_t>(qi));
            const int64_t gb = grow >> 5;
            if ((l32 & 15) == 0) st_dev(P.os16 + m * (N >> 4) + 2 * gb + (l32 >> 4), s);
            if (l32 == 0) {
                st_dev(P.od + m * (N >> 5) + gb, dd);
                st_dev(P.osumsq + m * (N >> 5) + gb, sq);
            }
        }
    }
}

// Positions staged in LDS at once (two rounds for M > 8; the raw weights
// stay in registers, so nothing is read twice from memory).
template <int M>
struct MG {
    static constexpr int value = M > 8 ? 8 : M;
};

// The rows, K chunk and matrix of a unit under the R-rows-per-lane layout:
// wave w takes rows [rw, rw + 32 / RS), rw = row0 + (32 / RS) (w % RS),
// over steps [w0, w1), the (w / RS)-th of SS parts of the chunk's steps.
struct UnitGeom {
    int tile, chunk, mat, c0, w0, w1, cs;
    int64_t row0, rw, s_begin;
};

template <int R>
__device__ __forceinline__ UnitGeom unit_geom(const PhaseDesc &P, int unit) {
    constexpr int RS = 4 / R, SS = 4 / RS;
    UnitGeom g;
    const int wave = threadIdx.x >> 6;
    g.tile = unit / P.per_tile;
    const int rem = unit % P.per_tile;
    g.chunk = rem % P.S;
    g.mat = rem / P.S;
    g.row0 = static_cast<int64_t>(g.tile) * kRows;
    const int64_t nsub = P.K >> 5;
    g.c0 = static_cast<int>(static_cast<int64_t>(g.chunk) * P.steps / P.S);
    const int c1 = static_cast<int>(static_cast<int64_t>(g.chunk + 1) * P.steps / P.S);
    const int tc = c1 - g.c0;
    g.w0 = g.c0 + (wave / RS) * tc / SS;
    g.w1 = g.c0 + (wave / RS + 1) * tc / SS;
    g.rw = g.row0 + (kRows / RS) * (wave % RS);
    g.s_begin = static_cast<int64_t>(g.c0) * 8;
    g.cs = static_cast<int>(min(static_cast<int64_t>(tc) * 8, nsub - g.s_begin));
    return g;
}

// Request every weight record of a unit (at most WS steps per
// wave and matrix) into raw.
// ALL: every record is written (steps a wave does not take re-read a
// record of its chunk), so no value of an earlier unit has to be kept.
template <int QT, int NM, bool ALL = false, int WS, int R>
__device__ __forceinline__ void issue_weights(WRaw<QT> (&raw)[NM][WS][R], const PhaseDesc &P,
                                              const UnitGeom &g) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 3, jl = lane & 7;
    const int64_t nsub = P.K >> 5;
    int64_t srow[R];
#pragma unroll
    for (int p = 0; p < R; p++) {
        int64_t rr = g.rw + grp * R + p;
        if (rr >= P.N) rr = 0;
        const int64_t sr = P.row_ids ? static_cast<int64_t>(gld(P.row_ids + rr)) : rr;
        // out-of-range ids are a caller error; clamp so no read leaves the matrix
        srow[p] = (sr < 0 || sr >= P.wrows) ? 0 : sr;
    }
#pragma unroll
    for (int mm = 0; mm < NM; mm++) {
        const uint8_t *__restrict__ w = P.w[g.mat + mm];
#pragma unroll
        for (int t = 0; t < WS; t++) {
            const int64_t sb = static_cast<int64_t>(g.w0 + t) * 8 + jl;
            if (ALL) {
                const int64_t sc = (g.w0 + t < g.w1 && sb < nsub) ? sb : static_cast<int64_t>(g.c0) * 8;
#pragma unroll
                for (int p = 0; p < R; p++) load_w<QT>(raw[mm][t][p], w, P, srow[p], sc);
            } else if (g.w0 + t < g.w1 && sb < nsub) {
#pragma unroll
                for (int p = 0; p < R; p++) load_w<QT>(raw[mm][t][p], w, P, srow[p], sb);
            }
        }
    }
}

// One unit: rows [row0, row0 + 32) x the K chunk `chunk`, for NM matrices
// from `mat` (NM = 2: both matrices of a gate/up pair, so the pair's
// product forms inside the unit).  Wave w takes rows [rw, rw + 32 / RS)
// over steps [w0, w1) of the chunk of each matrix (one step = 8 sub-blocks
// per row, one 256-element super-block of a K-quant); lane j of row group
// grp reads sub-block 8 t + j of rows rw + R grp + p, p < R.
// OWN: the unit requests its own weights first (raw is scratch); else raw
// already holds them (software-pipelined phases) and next >= 0 names the
// unit whose weights to request once the dot products are done.
template <int QT, int M, int NM, bool OWN>
__device__ __forceinline__ bool run_unit(const PhaseDesc &P, int unit,
                                         WRaw<QT> (&raw_in)[NM][Lay::WS][Lay::R],
                                         int next, uint8_t *act, float *ystage, float *wpart, float *parts, int CS,
                                         Shared<M> &sh, bool do_wait, bool timed, unsigned *status, bool restage) {
    constexpr int MGV = MG<M>::value;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 3, jl = lane & 7;
    const bool pair = P.ep_mode == SV_EP_PAIR;
    const int per_tile = P.per_tile;
    constexpr int kR = Lay::R, RS = Lay::RS, SS = Lay::SS, WS = Lay::WS;
    const UnitGeom g = unit_geom<kR>(P, unit);
    const int tile = g.tile, chunk = g.chunk, mat = g.mat;
    const int64_t row0 = g.row0;
    const int64_t nsub = P.K >> 5;
    const int w0 = g.w0, w1 = g.w1;
    const int64_t s_begin = g.s_begin;
    const int cs = g.cs;
    WRaw<QT> raw_own[NM][WS][kR];
    WRaw<QT>(&raw)[NM][WS][kR] = OWN ? raw_own : raw_in;
    if (OWN) issue_weights<QT, NM>(raw, P, g);
    // the epilogue's norm weight of this thread's row, fetched off the
    // critical path
    float g_row = 1.0f;
    if (P.gamma && P.ep_mode != SV_EP_NONE) {
        const int64_t gr = row0 + (threadIdx.x & 31);
        if (gr < P.N) g_row = gld(P.gamma + gr);
    }
    bool need_rs = false;
    if (do_wait) {
        if (P.wait && !wait_ready(P.wait, P.wait_target, status, sh.abort)) return false;
        if (timed && threadIdx.x == 0) {
            sh.t_wait = __builtin_amdgcn_s_memrealtime();
            sh.t_reduced = 0ull;
            sh.t_epi = 0ull;
        }
        need_rs = true;
    }
    float acc[NM][kR][M];
#pragma unroll
    for (int mm = 0; mm < NM; mm++)
#pragma unroll
        for (int p = 0; p < kR; p++)
#pragma unroll
            for (int m = 0; m < M; m++) acc[mm][p][m] = 0.0f;
#pragma unroll
    for (int m0 = 0; m0 < M; m0 += MGV) {
        const int mg = min(MGV, M - m0);
        // the chunk staged for the previous unit of this phase may be the
        // same one (then it is still in LDS)
        if (restage || M > MGV) {
            lds_barrier();
            if (m0 == 0 && need_rs && P.in_parts) rms_fetch(parts, P, M);
            stage_act(act, P, m0, mg, s_begin, cs, CS);
            // LDS transfers of this wave are complete once its loads are
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();
        }
        if (timed && m0 == 0 && threadIdx.x == 0) sh.t_staged = __builtin_amdgcn_s_memrealtime();
#pragma unroll
        for (int t = 0; t < WS; t++) {
            const int64_t sb = static_cast<int64_t>(w0 + t) * 8 + jl;
            if (w0 + t < w1 && sb < nsub) {
                const int sl = static_cast<int>(sb - s_begin);
#pragma unroll
                for (int mm = 0; mm < NM; mm++) {
                    WDec dec[kR];
#pragma unroll
                    for (int p = 0; p < kR; p++) decode_w<QT>(dec[p], raw[mm][t][p], jl);
#pragma unroll
                    for (int m = 0; m < MGV; m++) {
                        if (m0 + m < M) {
                            ARec ar;
                            read_act(ar, act + m * CS * kActRec, CS, sl);
                            const AExt ae = act_ext<QT>(ar);
#pragma unroll
                            for (int p = 0; p < kR; p++)
                                acc[mm][p][m0 + m] = block_term<QT>(dec[p], ar, ae, acc[mm][p][m0 + m]);
                        }
                    }
                }
            }
        }
    }
    if (timed && threadIdx.x == 0) sh.t_computed = __builtin_amdgcn_s_memrealtime();
    // The weight registers are free: the next unit's records are requested
    // now, so they stream in during this unit's reduction and epilogue.
    if (!OWN && next >= 0) issue_weights<QT, NM, true>(raw, P, unit_geom<kR>(P, next));
    // The input's RMS factors (first unit of a phase) are formed now, with
    // the weight registers free: their loads are in flight during the
    // reduction below.
    const bool rms = need_rs && P.in_parts;
    // Lanes of a row group: fixed-order sum; waves: partials through LDS,
    // added in wave order.
#pragma unroll
    for (int mm = 0; mm < NM; mm++)
#pragma unroll
        for (int p = 0; p < kR; p++)
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float v = group8_sum(acc[mm][p][m]);
                if (jl == 0)
                    wpart[((wave * NM + mm) * M + m) * kRows + (kRows / RS) * (wave % RS) + grp * kR + p] = v;
            }
    if (rms) {
        rms_store(parts, P, M, sh.rscale);
    } else if (need_rs && threadIdx.x < M) {
        sh.rscale[threadIdx.x] = 1.0f;
    }
    lds_barrier();
    // chunk value of (m, row): the SS step parts added in order, from waves
    // rs, rs + RS, ... of the row's part rs.  A tile is final here unless K
    // is split over units or a pair's matrices sit in two units.
    const bool split = P.S > 1 || (pair && NM == 1);
    for (int i = threadIdx.x; i < NM * M * kRows; i += kThreads) {
        const int mm = i / (M * kRows), r2 = i % (M * kRows), m = r2 / kRows, r = r2 % kRows;
        const int rs = r / (kRows / RS);
        float v = wpart[((rs * NM + mm) * M + m) * kRows + r];
#pragma unroll
        for (int sp = 1; sp < SS; sp++) v += wpart[(((sp * RS + rs) * NM + mm) * M + m) * kRows + r];
        if (!split) {
            ystage[((mat + mm) * M + m) * kRows + r] = v * sh.rscale[m];
        } else {
            const int64_t rr = row0 + r;
            if (rr < P.N)
                st_dev(P.partial + ((static_cast<int64_t>(mat + mm) * P.S + chunk) * M + m) * P.N + rr, v);
        }
    }
    if (!split) {
        lds_barrier();
        if (timed && threadIdx.x == 0) sh.t_reduced = __builtin_amdgcn_s_memrealtime();
        finish_tile<M>(P, ystage, row0, mat, mat + NM, NM == 2 || mat == P.ep_src, g_row, sh);
        if (timed && threadIdx.x == 0) sh.t_epi = __builtin_amdgcn_s_memrealtime();
        return true;
    }
    // K split over units: the last unit of the tile to finish adds the chunk
    // partials in chunk order and runs the epilogue.
    drain();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = add_dev(P.tile_count + tile, 1u);
        sh.last = (prev == static_cast<unsigned>(per_tile - 1)) ? 1 : 0;
    }
    lds_barrier();
    if (!sh.last) return true;
    const int rows_here = static_cast<int>(min(static_cast<int64_t>(kRows), static_cast<int64_t>(P.N) - row0));
    for (int i = threadIdx.x; i < P.n_w * M * kRows; i += kThreads) {
        const int mt = i / (M * kRows), r2 = i % (M * kRows), m = r2 / kRows, r = r2 % kRows;
        float s = 0.0f;
        if (r < rows_here) {
            const float *src = P.partial + (static_cast<int64_t>(mt) * P.S * M + m) * P.N + row0 + r;
            float v[kMaxS];
#pragma unroll
            for (int c = 0; c < kMaxS; c++) {
                // every chunk's partial is requested before any is used
                const float x = ld_dev(src + static_cast<int64_t>(c < P.S ? c : 0) * M * P.N);
                v[c] = c < P.S ? x : 0.0f;
            }
#pragma unroll
            for (int c = 0; c < kMaxS; c++)
                if (c < P.S) s += v[c];
        }
        ystage[(mt * M + m) * kRows + r] = s * sh.rscale[m];
    }
    if (threadIdx.x == 0)
        st_dev(P.tile_count + tile, 0u);
    lds_barrier();
    if (timed && threadIdx.x == 0) sh.t_reduced = __builtin_amdgcn_s_memrealtime();
    finish_tile<M>(P, ystage, row0, 0, P.n_w, true, g_row, sh);
    if (timed && threadIdx.x == 0) sh.t_epi = __builtin_amdgcn_s_memrealtime();
    return true;
}


// The units u, u + G, ... < nu of one phase on this workgroup.  A unit whose
// output the next phase reads is drained and counted; any other unit lets
// the next one's weights stream in during its own reduction and epilogue.
template <int QT, int M, int NM, bool PF>
__device__ __forceinline__ bool run_phase(const PhaseDesc &P, uint32_t u, uint32_t G, uint32_t nu, uint8_t *act,
                                          float *ystage, float *wpart, float *parts, int CS, Shared<M> &sh,
                                          unsigned *status, unsigned long long *tr) {
    WRaw<QT> raw[NM][Lay::WS][Lay::R];
    if (PF) issue_weights<QT, NM, true>(raw, P, unit_geom<Lay::R>(P, static_cast<int>(u)));
    bool first = true;
    int staged = -1;   // first step of the K chunk in LDS
    unsigned n_done = 0;
    for (; u < nu; u += G) {
        const int rem = static_cast<int>(u % P.per_tile);
        const int chunk = rem % P.S;
        const int c0 = static_cast<int>(static_cast<int64_t>(chunk) * P.steps / P.S);
        // Only units whose outputs the next phase reads are handed off
        // (drained and counted); the last phase has no reader at all.
        const bool counted = P.ready && (P.count_all || rem / P.S == P.ep_src);
        const bool more = u + G < nu;
        const int next = (PF && more && !counted) ? static_cast<int>(u + G) : -1;
        if (!run_unit<QT, M, NM, !PF>(P, static_cast<int>(u), raw, next, act, ystage, wpart, parts, CS, sh, first,
                                      first && tr != nullptr, status, c0 != staged))
            return false;
        staged = c0;
        n_done++;
        if (counted) drain();
        lds_barrier();
        if (counted && threadIdx.x < kReplicas)
            add_dev(P.ready + (threadIdx.x * kSlots + u % kSlots) * kSlotStride, 1u);
        if (threadIdx.x == 0) {
            sh.last = 0;
            if (first && tr) {
                tr[1] = sh.t_wait;
                tr[2] = sh.t_staged;
                tr[3] = sh.t_computed;
                tr[4] = __builtin_amdgcn_s_memrealtime();
                tr[7] = sh.t_reduced;
                tr[8] = sh.t_epi;
            }
        }
        first = false;
        lds_barrier();
        if (PF && more && next < 0)
            issue_weights<QT, NM, true>(raw, P, unit_geom<Lay::R>(P, static_cast<int>(u + G)));
    }
    if (tr && threadIdx.x == 0) {
        tr[5] = __builtin_amdgcn_s_memrealtime();
        tr[6] = n_done;
    }
    return true;
}

template <int M>
__device__ __forceinline__ bool dispatch_phase(const PhaseDesc &P, uint32_t u, uint32_t G, uint32_t nu, uint8_t *act,
                                               float *ystage, float *wpart, float *parts, int CS, Shared<M> &sh,
                                               unsigned *status, unsigned long long *tr) {
    // Phases with several units per workgroup and no reader (the head) run
    // software-pipelined: each unit's successor streams in during its
    // reduction and epilogue.
    if (!P.ready && u + G < nu) {
        if (P.qtype == SV_Q6_K)
            return run_phase<SV_Q6_K, M, 1, true>(P, u, G, nu, act, ystage, wpart, parts, CS, sh, status, tr);
        if (P.qtype == SV_Q8_0)
            return run_phase<SV_Q8_0, M, 1, true>(P, u, G, nu, act, ystage, wpart, parts, CS, sh, status, tr);
    }
    if (P.qtype == SV_Q4_K) {
        if (P.fused) return run_phase<SV_Q4_K, M, 2, false>(P, u, G, nu, act, ystage, wpart, parts, CS, sh, status, tr);
        return run_phase<SV_Q4_K, M, 1, false>(P, u, G, nu, act, ystage, wpart, parts, CS, sh, status, tr);
    }
    if (P.qtype == SV_Q6_K)
        return run_phase<SV_Q6_K, M, 1, false>(P, u, G, nu, act, ystage, wpart, parts, CS, sh, status, tr);
    return run_phase<SV_Q8_0, M, 1, false>(P, u, G, nu, act, ystage, wpart, parts, CS, sh, status, tr);
}

// Adds the workgroup's best (logit, index) keys of the phase to its argmax
// words.  In a pass those words are cleared by workgroup 0 at launch, so a
// workgroup waits for the flag that says so (set within microseconds of the
// start, long before any head tile is done; the wait is bounded like every
// other) before its first atomic maximum.
__device__ __forceinline__ void flush_best(const PhaseDesc &P, unsigned long long *best, int M,
                                           const unsigned *cleared, unsigned *status) {
    __syncthreads();
    if (P.argmax && static_cast<int>(threadIdx.x) < M) {
        if (cleared) {
            unsigned n = 0;
            while (ld_dev(cleared) == 0u) {
                __builtin_amdgcn_s_sleep(2);
                if (++n > kSpinLimit) {
                    or_dev(status, 2u);
                    break;
                }
            }
        }
        if (best[threadIdx.x]) max_dev(P.argmax + threadIdx.x, best[threadIdx.x]);
        best[threadIdx.x] = 0ull;
    }
    __syncthreads();
}

// LDS layout of a workgroup: act chunk [MG][CS * kActRec] | ystage
// [3][M][kRows] fp32 | wave partials [4][2][M][kRows] fp32 | the input's
// sums of squares [M][n_parts] fp32.
template <int M>
__device__ __forceinline__ void lds_parts(uint8_t *smem, int CS, float *&ystage, float *&wpart, float *&parts) {
    ystage = reinterpret_cast<float *>(smem + MG<M>::value * CS * kActRec);
    wpart = ystage + 3 * M * kRows;
    parts = wpart + 8 * M * kRows;
}

// One workgroup per unit of a single phase.
template <int M>
__global__ __launch_bounds__(kThreads, M <= 8 ? 2 : 1) void phase_kernel(PhaseDesc P, int CS) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ Shared<M> sh;
    float *ystage, *wpart, *parts;
    lds_parts<M>(smem, CS, ystage, wpart, parts);
    if (threadIdx.x < SV_MAX_M) sh.best[threadIdx.x] = 0ull;
    dispatch_phase<M>(P, blockIdx.x, gridDim.x, static_cast<uint32_t>(P.n_units), smem, ystage, wpart, parts, CS, sh,
                      nullptr, nullptr);
    flush_best(P, sh.best, M, nullptr, nullptr);
}

// ctl: control words (kCtl*), then per phase kPhaseCounters counters of
// finished units, kSlotStride words apart.  The last workgroup to exit
// adds the run's status to kCtlResult (an OR the host reads and clears) and
// returns every other word to zero (and, after an expired wait, the tile counters of split tiles), so
// the next run starts clean without a reset launch.
template <int M>
__global__ __launch_bounds__(kThreads, M <= 8 ? 2 : 1) void pass_kernel(const PhaseDesc *__restrict__ table, int n_phases,
                                                        unsigned *ctl, int CS, ArgmaxList am,
                                                        unsigned long long *trace) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ Shared<M> sh;
    __shared__ PhaseDesc P;
    float *ystage, *wpart, *parts;
    lds_parts<M>(smem, CS, ystage, wpart, parts);
    unsigned *status = ctl + kCtlStatus;
    const unsigned *cleared = ctl + kCtlArgmaxClear;
    if (threadIdx.x < SV_MAX_M) sh.best[threadIdx.x] = 0ull;
    // Workgroup 0 clears every argmax of the pass, waits until the stores
    // are done and raises the flag flush_best waits on.
    if (blockIdx.x == 0 && am.n > 0) {
        for (int i = 0; i < am.n; i++)
            if (static_cast<int>(threadIdx.x) < am.M[i]) st_dev(am.p[i] + threadIdx.x, 0ull);
        drain();
        __syncthreads();
        if (threadIdx.x == 0) st_dev(ctl + kCtlArgmaxClear, 1u);
    }
    const uint32_t G = gridDim.x, b = blockIdx.x;
    int cur = -1;
    bool ok = true;
    for (int p = 0; p < n_phases && ok; p++) {
        // units of phase p are dealt round-robin, continuing where phase
        // p-1 stopped, so every workgroup gets its share of every phase
        const uint32_t base = table[p].unit_base, nu = static_cast<uint32_t>(table[p].n_units);
        uint32_t u = (b + G - base % G) % G;
        if (u >= nu) continue;
        if (cur >= 0) flush_best(P, sh.best, M, cleared, status);
        if (threadIdx.x == 0) P = table[p];
        __syncthreads();
        cur = p;
        unsigned long long *tr = trace ? trace + (static_cast<size_t>(b) * n_phases + p) * kTraceWords : nullptr;
        if (tr && threadIdx.x == 0) {
            tr[0] = __builtin_amdgcn_s_memrealtime();
            // where the workgroup runs: HW_ID (CU, shader array and engine
            // fields) and XCC_ID, full 32-bit reads of the two registers
            tr[9] = static_cast<unsigned long long>(__builtin_amdgcn_s_getreg(0xF804)) |
                    (static_cast<unsigned long long>(__builtin_amdgcn_s_getreg(0xF814)) << 32);
        }
        ok = dispatch_phase<M>(P, u, G, nu, smem, ystage, wpart, parts, CS, sh, status, tr);
    }
    if (cur >= 0) flush_best(P, sh.best, M, cleared, status);
    drain();
    __syncthreads();
    if (threadIdx.x == 0) sh.last = (add_dev(ctl + kCtlExited, 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    if (sh.last) {
        const unsigned st = ld_dev(status);
        for (int i = 1 + static_cast<int>(threadIdx.x); i < 1 + n_phases * kPhaseCounters; i += kThreads)
            st_dev(ctl + i * kSlotStride, 0u);
        if (st != 0u) {
            // an aborted run can leave split tiles partly counted
            for (int p = 0; p < n_phases; p++) {
                unsigned *tc = table[p].tile_count;
                if (!tc) continue;
                for (int t = static_cast<int>(threadIdx.x); t < table[p].n_tiles; t += kThreads) st_dev(tc + t, 0u);
            }
        }
        if (threadIdx.x == 0) {
            if (st != 0u) or_dev(ctl + kCtlResult, st);
            st_dev(ctl + kCtlStatus, 0u);
            st_dev(ctl + kCtlExited, 0u);
            st_dev(ctl + kCtlArgmaxClear, 0u);
        }
    }
}
}  // namespace sv
