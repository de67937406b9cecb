// matvec_dev.h - device code of the verification projection (a3), its
// fused producer epilogue (a4), the output head with fused argmax (a6, a9)
// and the phase sequencing of a whole pass in one persistent launch (a5).
// Included by matvec_inst.hip only, which instantiates the kernels for one M.
//
// One weight stream serves all M positions ("Inside OpenJet Engine: making
// speculative decoding pay", section "One GPU launch for a speculative
// cycle": weight reads serve multiple verification positions, activation
// loads are reused across weight rows, and one launch carries the phases of
// a cycle separated by synchronisation between phases).
//
// Work decomposition.  A phase (one to three matrices sharing an input) is
// cut into units = (32-row tile, K chunk, matrix); for M <= 8 a unit of a
// gate/up pair covers both matrices (their items alternate in the ring and
// the product forms in the control wave), above that each matrix is a unit
// of its own and the values meet in the tile's last unit.  K is walked in steps of 256 elements (one K-quant super-block,
// eight Q8_0 blocks); a chunk is at most 20 steps (5120 elements), so
// S(K) = ceil(steps / 20) depends on K alone.
//
// Roles in a workgroup.  Eight compute waves and one control wave.
//  * Compute wave w takes the 16-row half tile w & 1 over the quarter
//    w >> 1 of the chunk's steps.  Lane j of an 8-lane row group reads sub-block
//    8t + j of two rows, so a group reads 128 contiguous bytes of a row, and
//    each record is reused from registers for all M positions.  A compute
//    wave requests its weights through a ring of items held in registers
//    (two to four, by M): the next free item is requested as soon as
//    an item's dot products are done, across unit and phase boundaries, so
//    a compute wave never waits for a store or a hand-off and its loads keep
//    streaming while the control wave synchronises.  At the end of a unit
//    the wave writes its per-row partial sums to LDS.  The two compute
//    waves of a SIMD (w and w + 4) raise their priority in turns, two items
//    of a unit each, the younger first, so they finish a unit together.
//  * The control wave never loads weights.  It waits for the phase that
//    writes a unit's input, stages the input chunk into LDS with
//    load-to-LDS transfers, forms the input's RMS factors, adds the compute
//    waves' partial sums, runs the epilogue (outputs, argmax candidates,
//    requantisation of the next input), and hands the unit off.  Its memory
//    counter covers only its own transfers and stores, so a hand-off waits
//    for nothing but the unit's outputs.
// Arithmetic.  Integer block sums come from v_dot4 (exact); each block's
// fp32 combine is a fixed sequence of operations per (row, position); a lane
// adds its blocks in increasing order, the 8 lanes of a group are combined
// in a fixed DPP tree, the four step quarters in order and the K chunks in
// chunk order.  Nothing depends on M or on which workgroup ran which unit,
// so every output row is bit-identical to the same row computed alone, and
// runs are deterministic.
// Scheduling.  A pass runs as one persistent launch sized to the number of
// workgroups the GPU holds at once; the units of each phase are dealt
// round-robin, continuing where the previous phase stopped.  A single call
// launches one workgroup per unit.  Every wait is bounded.
#pragma once

#include "matvec_launch.h"

namespace sv {

#define SV_AS3 __attribute__((address_space(3)))
#define SV_AS4 __attribute__((address_space(4)))

constexpr int kCompWaves = 8;
constexpr int kStepParts = kCompWaves / 2;   // compute waves per half tile

// Ring depth (items in flight per compute wave) by M: deeper rings for few
// positions, where a wave's dot products leave registers free.  It changes
// no result.
template <int M>
struct RingDepth {
#ifdef SV_RING
    static constexpr int value = SV_RING;
#else
    static constexpr int value = M == 1 ? 5 : (M <= 2 ? 4 : (M <= 5 ? 3 : 2));
#endif
};

// ------------------------------------------------------------ tables
// Phase descriptors are read with scalar loads: from the pass's table in
// device memory through a constant-address-space pointer, or from the
// kernel argument of a single call.  A cursor walks the units a workgroup
// runs: in a pass the host's schedule lists them, per workgroup and in
// phase order (entry = phase << 20 | unit); in a single call workgroup b
// runs unit b.
struct UnitCur {
    int p;
    uint32_t u;
    uint32_t i, end;   // the workgroup's schedule entries [i, end) (pass)
};

// Scalar: the phase and list indices are wave-uniform, so the table and the
// lists can be read with scalar loads through the scalar cache.  That
// shortens the per-unit table reads, which set the pace at one row (units
// are short there); with more rows the same pass measured slower with
// scalar reads, so they are taken at M = 1 only.
template <bool Scalar>
struct ManyTab {
    const SV_AS4 PhaseDesc *t;
    const SV_AS4 uint32_t *sched;   // [G + 1] entry offsets per workgroup, then the entries
    int n;
    uint32_t G;
    static __device__ __forceinline__ int uni(int i) { return Scalar ? __builtin_amdgcn_readfirstlane(i) : i; }
    __device__ __forceinline__ const SV_AS4 PhaseDesc &operator[](int p) const { return t[uni(p)]; }
    __device__ __forceinline__ void decode(UnitCur &c) const {
        if (c.i < c.end) {
            const uint32_t e = sched[G + 1 + static_cast<uint32_t>(uni(static_cast<int>(c.i)))];
            c.p = static_cast<int>(e >> 20);
            c.u = e & 0xFFFFFu;
        } else {
            c.p = n;
        }
    }
    __device__ __forceinline__ void first(uint32_t b, UnitCur &c) const {
        c.i = sched[b];
        c.end = sched[b + 1];
        decode(c);
    }
    __device__ __forceinline__ void next(UnitCur &c) const {
        c.i++;
        decode(c);
    }
};
// The single call's one phase, read where the launch argument lies (the
// kernel argument segment, through scalar loads): a copy in the kernel would
// be addressed by runtime indices (the matrix of a unit) and so live in
// scratch memory.
struct OneTab {
    const SV_AS4 PhaseDesc *t;
    __device__ __forceinline__ const SV_AS4 PhaseDesc &operator[](int) const { return *t; }
    __device__ __forceinline__ void first(uint32_t b, UnitCur &c) const {
        c.u = b;
        c.p = b < static_cast<uint32_t>(t->n_units) ? 0 : 1;
    }
    __device__ __forceinline__ void next(UnitCur &c) const { c.p = 1; }   // one unit per workgroup
};

template <class Tab>
__device__ __forceinline__ void unit_first(const Tab &tab, int, uint32_t b, uint32_t, UnitCur &c) {
    tab.first(b, c);
}
template <class Tab>
__device__ __forceinline__ void unit_next(const Tab &tab, int, uint32_t, uint32_t, UnitCur &c) {
    tab.next(c);
}

// Geometry of a unit: tile, K chunk (of the tile's nch) and matrix; the
// chunk's steps [c0, c1) and its sub-blocks [s_begin, s_begin + cs).
// Units [0, T1 per_tile) are the tiles cut into S chunks, tile-major, then
// matrix, then chunk.  The rest are the tiles cut into S1 = f S chunks,
// ordered so that, with the phase starting on a round, the workgroup that
// ran chunk c of the first kind (unit index = c mod S, matrix likewise) gets
// one of the f finer chunks inside chunk c.
struct UnitPos {
    int tile, chunk, nch, mat, c0, c1, s_begin, cs;
    int pb, pcs;   // sub-blocks of the unit's K chunk at S chunks per tile (what is staged)
};
__device__ __forceinline__ uint32_t fdiv(uint32_t n, uint32_t m, uint32_t sh) {
    return static_cast<uint32_t>((static_cast<uint64_t>(n) * m) >> sh);
}
template <class PD>
__device__ __forceinline__ UnitPos unit_pos(const PD &P, uint32_t u) {
    UnitPos g;
    const uint32_t per_tile = P.per_tile, S = P.S, steps = P.steps;
    const uint32_t head = static_cast<uint32_t>(P.T1) * per_tile;
    const bool tail = u >= head;
    const uint32_t v = tail ? u - head : u;
    const uint32_t q = fdiv(v, P.div_pt.m, P.div_pt.sh), rem = v - q * per_tile;
    const uint32_t mat = fdiv(rem, P.div_S.m, P.div_S.sh), c = rem - mat * S;
    g.mat = static_cast<int>(mat);
    const int nsub = P.K >> 5;
    {
        // the chunk of S the unit lies in (its own chunk unless the tile is
        // cut finer): staging it serves every unit of that chunk
        const int p0 = static_cast<int>(fdiv(c * steps, P.div_S.m, P.div_S.sh));
        const int p1 = static_cast<int>(fdiv((c + 1) * steps, P.div_S.m, P.div_S.sh));
        g.pb = p0 * 8;
        g.pcs = min((p1 - p0) * 8, nsub - g.pb);
    }
    uint32_t nch = S, chunk = c, tile = q;
    if (tail) {
        const uint32_t f = fdiv(static_cast<uint32_t>(P.S1), P.div_S.m, P.div_S.sh);
        const uint32_t qf = fdiv(q, P.div_f.m, P.div_f.sh);
        chunk = f * c + (q - qf * f);
        tile = static_cast<uint32_t>(P.T1) + qf;
        nch = P.S1;
    }
    g.tile = static_cast<int>(tile);
    g.chunk = static_cast<int>(chunk);
    g.nch = static_cast<int>(nch);
    const uint32_t dm = tail ? P.div_S1.m : P.div_S.m, ds = tail ? P.div_S1.sh : P.div_S.sh;
    g.c0 = static_cast<int>(fdiv(chunk * steps, dm, ds));
    g.c1 = static_cast<int>(fdiv((chunk + 1) * steps, dm, ds));
    g.s_begin = g.c0 * 8;
    g.cs = min((g.c1 - g.c0) * 8, nsub - g.s_begin);
    return g;
}

// Steps [w0, w1) of compute wave `wave`, and the number of ring items they
// make (at least one: a wave with no step still passes through the unit).
// A Q4_K record of one matrix is 5 words, so its items carry two steps.
struct WaveSpan {
    int w0, w1, sp, nh, nitems;   // nh items per matrix
};
template <class PD>
__device__ __forceinline__ WaveSpan wave_span(const PD &P, const UnitPos &g, int wave) {
    WaveSpan s;
    const int tc = g.c1 - g.c0, part = wave >> 1;
    s.w0 = g.c0 + part * tc / kStepParts;
    s.w1 = g.c0 + (part + 1) * tc / kStepParts;
    s.sp = P.qtype == SV_Q4_K ? 2 : 1;
    // a fused pair runs the gate items, then the up items, over the same
    // steps (one set of accumulators serves both in turn)
    s.nh = max(1, (s.w1 - s.w0 + s.sp - 1) >> (s.sp - 1));
    s.nitems = s.nh * (P.fused ? 2 : 1);
    return s;
}

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

// One item of the ring: the raw records of a lane in named registers (every
// index below is a template parameter, so nothing is ever addressed by a
// runtime index, which would put the ring in memory).  An item is always the
// same eight loads into the same registers, four of 16 bytes (quads q0-q3)
// and four of 4 bytes (words x0-x3); only their addresses depend on the
// format.  So the loads in flight never depend on the path taken, and the
// compiler's wait before a slot is read covers that slot alone.
//   Q4_K (record i = 2 step + row): quants in quad i, the lane's header
//        dword (lane & 3) in word i
//   Q6_K (row p < 2): low nibbles in quad p, high bits in the first 8 bytes
//        of quad 2 + p, the two int8 sub-scales in word p, d in word 2 + p
//   Q8_0 (row p < 2): quants in quads 2p and 2p + 1, d in word p
// (a Q6_K or Q8_0 word is the dword of the row's pair; the row's 2 bytes
// are its half hs[p] / 16)
// Words a format does not use repeat an earlier address.
struct Slot {
    uint4 q0, q1, q2, q3;
    uint32_t x0, x1, x2, x3;
};

template <int I>
__device__ __forceinline__ const uint4 &quad(const Slot &s) {
    if constexpr (I == 0) return s.q0;
    else if constexpr (I == 1) return s.q1;
    else if constexpr (I == 2) return s.q2;
    else return s.q3;
}
template <int I>
__device__ __forceinline__ uint32_t word(const Slot &s) {
    if constexpr (I == 0) return s.x0;
    else if constexpr (I == 1) return s.x1;
    else if constexpr (I == 2) return s.x2;
    else return s.x3;
}

template <int QT, int I>
__device__ __forceinline__ WRaw<QT> rec_of(const Slot &s, uint32_t hs) {
    WRaw<QT> r;
    if constexpr (QT == SV_Q8_0) {
        r.q0 = quad<2 * I>(s);
        r.q1 = quad<2 * I + 1>(s);
        r.d = word<I>(s) >> hs;
    } else if constexpr (QT == SV_Q4_K) {
        r.q = quad<I>(s);
        r.h = word<I>(s);
    } else {
        r.l = quad<I>(s);
        const uint4 hq = quad<2 + I>(s);
        r.h = make_uint2(hq.x, hq.y);
        r.sc = word<I>(s) >> hs;
        r.d = word<2 + I>(s) >> hs;
    }
    return r;
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

// LDS layout of a staged chunk of cs sub-blocks of all M positions, with
// R = row_sub<M>(cs) (kRowSub, or cs at M = 1): codes [M][R][32] (the global
// bytes as they are), scales [M][R] fp32, code sums [M][R][2] int32, each
// position's row holding the chunk's cs records first; where they are
// staged, the RMS partials of the input follow, [M][n_parts].
struct ActLds {
    const uint8_t *q;
    const float *d;
    const int2 *x;
    int begin;   // first staged sub-block of K
};
template <int M>
__device__ __forceinline__ ActLds act_lds(const uint8_t *act, int cs, int begin) {
    ActLds a;
    a.begin = begin;
    a.q = act;
    a.d = reinterpret_cast<const float *>(act + M * row_sub<M>(cs) * 32);
    a.x = reinterpret_cast<const int2 *>(act + M * row_sub<M>(cs) * 36);
    return a;
}
// With several positions, every position's row of a field starts kRowSub
// records after the previous one whatever the chunk's length, so a
// position's offset is a constant of the instruction and only the
// sub-block's address is computed.
__device__ __forceinline__ void read_act(ARec &r, const ActLds &A, int m, int sl) {
    const uint8_t *q = A.q + (m * kRowSub + sl) * 32;
    const uint4 lo = *reinterpret_cast<const uint4 *>(q);
    const uint4 hi = *reinterpret_cast<const uint4 *>(q + 16);
    r.v[0] = lo.x; r.v[1] = lo.y; r.v[2] = lo.z; r.v[3] = lo.w;
    r.v[4] = hi.x; r.v[5] = hi.y; r.v[6] = hi.z; r.v[7] = hi.w;
    r.d = A.d[m * kRowSub + sl];
    const int2 x = A.x[m * kRowSub + sl];
    r.x0 = x.x;
    r.x1 = x.y;
}

// ------------------------------------------------------------ lane sums
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
// Reductions over the 32 lanes of a half-wave (every lane gets the result):
// within each row of 16 by DPP, then the two rows by one lane exchange.
// The two 16-lane rows of each half-wave side by side: v_permlane16_swap
// with v in both operands leaves rows (0, 0, 2, 2) in the first result and
// (1, 1, 3, 3) in the second, so a symmetric combine of the two gives each
// lane the value of its row pair, with no LDS round trip.
struct RowPair {
    uint32_t a, b;
};
__device__ __forceinline__ RowPair row_pair(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return {static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1])};
}
__device__ __forceinline__ float half_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x128>(v));
    const RowPair p = row_pair(__float_as_uint(v));
    return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ float half_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x128>(v);
    const RowPair p = row_pair(__float_as_uint(v));
    return __uint_as_float(p.a) + __uint_as_float(p.b);
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
    const RowPair lo = row_pair(static_cast<uint32_t>(v & 0xFFFFFFFFull));
    const RowPair hi = row_pair(static_cast<uint32_t>(v >> 32));
    return umax64((static_cast<unsigned long long>(hi.a) << 32) | lo.a,
                  (static_cast<unsigned long long>(hi.b) << 32) | lo.b);
}

// Workgroup barrier for LDS data only: waits for this wave's LDS
// operations, not for its outstanding global loads (a full __syncthreads
// would also wait for the weight records already requested).  No global
// memory written before it is read by another wave after it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------ shared state
template <int M>
struct Shared {
    float rscale[SV_MAX_M];
    unsigned long long best[SV_MAX_M];
    unsigned abort;
    int stb, stc;   // staged sub-blocks [stb, stb + stc), published before B1
};

// Dynamic LDS: wave partials [2 buffers][8 waves][NMat][M][16 rows] fp32
// (two matrices where a unit may cover a fused pair, M <= 8), then the
// staged input chunk.
template <int M>
struct NMat {
    static constexpr int value = M <= 8 ? 2 : 1;
};
template <int M>
__device__ __forceinline__ float *wpart_buf(uint8_t *smem, int buf) {
    return reinterpret_cast<float *>(smem) + buf * (kCompWaves * NMat<M>::value * M * 16);
}
template <int M>
__device__ __forceinline__ uint8_t *act_base(uint8_t *smem) {
    return smem + 2 * kCompWaves * NMat<M>::value * M * 16 * 4;
}

// Trace record of a (workgroup, phase), kTraceWords words written by the
// control wave: real-time counter at the first unit of the phase, input
// ready, input staged, first unit computed, first unit handed off, last unit
// handed off; units run; first unit combined, its outputs written;
// HW_ID | XCC_ID << 32; its partial sums landed, its outputs landed;
// staging transfers issued, landed; two unused words.
__device__ __forceinline__ unsigned long long now() { return __builtin_amdgcn_s_memrealtime(); }

// ============================================================ compute waves
// The item cursor of a compute wave: unit, its geometry, the item inside
// it, and the phase fields the loads and the dot products need.
struct ItemCur {
    UnitCur uc;
    int item;
    // phase
    const uint8_t *w0, *w1, *w2;
    const uint8_t *wm;   // matrix of the current unit
    int qtype, fused, K, N, wrows;
    uint32_t bbytes;   // bytes of a weight block
    uint32_t sp;       // steps per item (2 for Q4_K)
    uint32_t last;     // the last step an item of this wave may read
    const int32_t *row_ids;
    // unit
    UnitPos g;
    WaveSpan s;
    bool newphase;    // the unit opens a phase (a barrier opens it)
    uint32_t off[8];  // this lane's byte offsets of the unit's eight loads (load cursor only)
    uint32_t hs[2];   // 16 x (row & 1) of this lane's two rows (compute cursor only)
};

template <class Tab>
__device__ __forceinline__ void cur_phase(const Tab &tab, ItemCur &c) {
    const auto &P = tab[c.uc.p];
    c.w0 = P.w[0];
    c.w1 = P.w[1];
    c.w2 = P.w[2];
    c.qtype = P.qtype;
    c.fused = P.fused;
    c.K = P.K;
    c.N = P.N;
    c.wrows = P.wrows;
    c.bbytes = P.bbytes;
    c.sp = P.qtype == SV_Q4_K ? 2u : 1u;
    c.row_ids = P.row_ids;
}

// Rows of this lane in the unit: 2 grp + p of the wave's half tile, mapped
// through row_ids (read with scalar loads, so they never wait on the ring's
// weight records) and clamped into the matrix.
__device__ __forceinline__ void lane_rows(const ItemCur &c, int wave, int32_t (&rho)[2]) {
    const int lane = threadIdx.x & 63, grp = lane >> 3;
    const int64_t rw = static_cast<int64_t>(c.g.tile) * kRows + 16 * (wave & 1);
    if (c.row_ids) {
        const SV_AS4 int32_t *ids = reinterpret_cast<const SV_AS4 int32_t *>(reinterpret_cast<uintptr_t>(c.row_ids));
        int32_t id[16];
#pragma unroll
        for (int k = 0; k < 16; k++) {
            const int64_t r = rw + k;
            id[k] = ids[r < c.N ? r : 0];
        }
#pragma unroll
        for (int p = 0; p < 2; p++) {
            int32_t v = id[p];
#pragma unroll
            for (int k = 1; k < 8; k++)
                if (grp == k) v = id[2 * k + p];
            rho[p] = (v < 0 || v >= c.wrows) ? 0 : v;
        }
    } else {
        // rows of the last half tile past the matrix are zero in the layout;
        // a half tile wholly past it reads row 0 (its outputs are dropped)
        const int64_t padded = ((static_cast<int64_t>(c.wrows) + 15) >> 4) << 4;
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const int64_t r = rw + grp * 2 + p;
            rho[p] = static_cast<int32_t>(r < padded ? r : 0);
        }
    }
}

// The compute cursor needs only which half of a pair dword holds each row.
__device__ __forceinline__ void cur_shifts(ItemCur &c, int wave) {
    if (c.row_ids) {
        int32_t rho[2];
        lane_rows(c, wave, rho);
        c.hs[0] = static_cast<uint32_t>(rho[0] & 1) * 16u;
        c.hs[1] = static_cast<uint32_t>(rho[1] & 1) * 16u;
    } else {
        c.hs[0] = 0u;    // rows 2 g and 2 g + 1 of the half tile
        c.hs[1] = 16u;
    }
}

__device__ __forceinline__ void cur_rows(ItemCur &c, int wave) {
    const int lane = threadIdx.x & 63, jl = lane & 7;
    int32_t rho[2];
    lane_rows(c, wave, rho);
    // byte offset of each row's half-tile block column, then of the pieces
    const uint32_t steps = static_cast<uint32_t>((c.K + 255) >> 8);
    uint32_t hb[2];
    int rr[2];
#pragma unroll
    for (int p = 0; p < 2; p++) {
        hb[p] = static_cast<uint32_t>(rho[p] >> 4) * steps * c.bbytes;
        rr[p] = rho[p] & 15;
    }
    if (c.qtype == SV_Q4_K) {
        c.off[0] = hb[0] + blk_q4k_codes(rr[0], jl);
        c.off[1] = hb[1] + blk_q4k_codes(rr[1], jl);
        c.off[2] = c.off[0];
        c.off[3] = c.off[1];
        c.off[4] = hb[0] + blk_q4k_hdr(rr[0]) + (lane & 3) * 4;
        c.off[5] = hb[1] + blk_q4k_hdr(rr[1]) + (lane & 3) * 4;
        c.off[6] = c.off[4];
        c.off[7] = c.off[5];
    } else if (c.qtype == SV_Q6_K) {
        c.off[0] = hb[0] + blk_q6k_ql(rr[0], jl);
        c.off[1] = hb[1] + blk_q6k_ql(rr[1], jl);
        c.off[2] = hb[0] + blk_q6k_qh(rr[0], jl);
        c.off[3] = hb[1] + blk_q6k_qh(rr[1], jl);
        c.off[4] = hb[0] + blk_q6k_sc(rr[0], jl);
        c.off[5] = hb[1] + blk_q6k_sc(rr[1], jl);
        c.off[6] = hb[0] + blk_q6k_d(rr[0]);
        c.off[7] = hb[1] + blk_q6k_d(rr[1]);
    } else {
        c.off[0] = hb[0] + blk_q80_lo(rr[0], jl);
        c.off[1] = c.off[0] + 1024u;
        c.off[2] = hb[1] + blk_q80_lo(rr[1], jl);
        c.off[3] = c.off[2] + 1024u;
        c.off[4] = hb[0] + blk_q80_d(rr[0], jl);
        c.off[5] = hb[1] + blk_q80_d(rr[1], jl);
        c.off[6] = c.off[4];
        c.off[7] = c.off[5];
    }
}

template <class Tab>
__device__ __forceinline__ void cur_unit(const Tab &tab, ItemCur &c, int wave, bool phase_changed, bool rows) {
    const auto &P = tab[c.uc.p];
    c.g = unit_pos(P, c.uc.u);
    c.s = wave_span(P, c.g, wave);
    c.last = static_cast<uint32_t>(max(c.s.w1 - 1, c.g.c0));
    c.item = 0;
    c.newphase = phase_changed;
    // integer arithmetic, not a select: a select among the three fields is
    // turned into an indexed load, which puts the whole cursor in memory
    const uint64_t m0 = c.g.mat == 0, m1 = c.g.mat == 1, m2 = c.g.mat == 2;
    c.wm = reinterpret_cast<const uint8_t *>(m0 * reinterpret_cast<uint64_t>(c.w0) +
                                             m1 * reinterpret_cast<uint64_t>(c.w1) +
                                             m2 * reinterpret_cast<uint64_t>(c.w2));
    if (rows) cur_rows(c, wave);
    else cur_shifts(c, wave);
}

template <class Tab>
__device__ __forceinline__ bool cur_init(const Tab &tab, int n_phases, uint32_t b, uint32_t G, ItemCur &c, int wave,
                                         bool rows) {
    unit_first(tab, n_phases, b, G, c.uc);
    if (c.uc.p >= n_phases) return false;
    cur_phase(tab, c);
    cur_unit(tab, c, wave, true, rows);
    return true;
}

// Next item; false at the end of the workgroup's units.
template <class Tab>
__device__ __forceinline__ bool cur_advance(const Tab &tab, int n_phases, uint32_t b, uint32_t G, ItemCur &c,
                                            int wave, bool rows) {
    if (++c.item < c.s.nitems) return true;
    const int p0 = c.uc.p;
    unit_next(tab, n_phases, b, G, c.uc);
    if (c.uc.p >= n_phases) return false;
    if (c.uc.p != p0) cur_phase(tab, c);
    cur_unit(tab, c, wave, c.uc.p != p0, rows);
    return true;
}

// Like cur_advance, but at the end of the sequence the cursor stays on the
// last item (the load cursor then re-reads it; see ring_step).
template <class Tab>
__device__ __forceinline__ bool cur_advance_keep(const Tab &tab, int n_phases, uint32_t b, uint32_t G, ItemCur &c,
                                                 int wave, bool rows) {
    if (c.item + 1 < c.s.nitems) {
        c.item++;
        return true;
    }
    UnitCur nx = c.uc;
    unit_next(tab, n_phases, b, G, nx);
    if (nx.p >= n_phases) return false;
    const int p0 = c.uc.p;
    c.uc = nx;
    if (c.uc.p != p0) cur_phase(tab, c);
    cur_unit(tab, c, wave, c.uc.p != p0, rows);
    return true;
}

// Requests the records of the cursor's item into slot s: eight loads at a
// wave-uniform block address (scalar registers) plus the lane's offsets of
// the unit.  Every item issues the same loads whether or not its steps
// exist (a step past the wave's span reads the last step of the span again,
// or the chunk's first step for an empty span, and is never used), so the
// number of loads in flight does not depend on the data.
__device__ __forceinline__ uint4 q16(const uint8_t *p) { return gld16_nt(p); }
__device__ __forceinline__ uint32_t w4(const uint8_t *p) { return gld(reinterpret_cast<const uint32_t *>(p)); }

__device__ __forceinline__ void load_item(Slot &s, const ItemCur &c) {
    // integer arithmetic on wave-uniform fields only (no booleans), so the
    // block addresses stay in scalar registers: a fused pair's items
    // [0, nh) are gate, [nh, 2 nh) up, over the same steps
    const uint32_t item = static_cast<uint32_t>(c.item), nh = static_cast<uint32_t>(c.s.nh);
    const uint32_t odd = item >= nh ? 1u : 0u, it = item - odd * nh;
    const uint32_t t0 = min(static_cast<uint32_t>(c.s.w0) + it * c.sp, c.last);
    const uint32_t t1 = min(t0 + c.sp - 1u, c.last);
    const uint64_t wm = reinterpret_cast<uint64_t>(c.wm), w1 = reinterpret_cast<uint64_t>(c.w1);
    const uint64_t wsel = wm + static_cast<uint64_t>(odd) * (w1 - wm);
    const uint8_t *b0 = reinterpret_cast<const uint8_t *>(wsel + static_cast<uint64_t>(t0 * c.bbytes));
    const uint8_t *b1 = reinterpret_cast<const uint8_t *>(wsel + static_cast<uint64_t>(t1 * c.bbytes));
    s.q0 = q16(b0 + c.off[0]);
    s.q1 = q16(b0 + c.off[1]);
    s.q2 = q16(b1 + c.off[2]);
    s.q3 = q16(b1 + c.off[3]);
    s.x0 = w4(b0 + c.off[4]);
    s.x1 = w4(b0 + c.off[5]);
    s.x2 = w4(b1 + c.off[6]);
    s.x3 = w4(b1 + c.off[7]);
}

// The block terms of one step (sub-block sl of the staged chunk) for the
// two rows whose records are I0 and I0 + 1 of the slot, into acc[p][*].
template <int QT, int I0, int M>
__device__ __forceinline__ void step_terms(const Slot &s, const ActLds &A, int sl, float (&acc)[2][M],
                                           uint32_t hs0, uint32_t hs1) {
    const int jl = threadIdx.x & 7;
    // up to M = 8 the activation record of position m + 1 is read while
    // position m is computed, and the first one while the weights are
    // decoded, so the LDS latency hides behind arithmetic (above that the
    // second record's registers are not free)
    constexpr bool kPipe = M <= 8;
    ARec cur;
    read_act(cur, A, 0, sl);
    WDec d0, d1;
    decode_w<QT>(d0, rec_of<QT, I0>(s, hs0), jl);
    decode_w<QT>(d1, rec_of<QT, I0 + 1>(s, hs1), jl);
#pragma unroll
    for (int m = 0; m < M; m++) {
        ARec nxt;
        if constexpr (kPipe) {
            if (m + 1 < M) read_act(nxt, A, m + 1, sl);
            // keep the reads above the arithmetic that does not need them
            __builtin_amdgcn_sched_barrier(0);
        } else if (m > 0) {
            read_act(cur, A, m, sl);
        }
        const AExt ae = act_ext(cur);
        acc[0][m] = block_term<QT>(d0, cur, ae, acc[0][m]);
        acc[1][m] = block_term<QT>(d1, cur, ae, acc[1][m]);
        if constexpr (kPipe)
            if (m + 1 < M) cur = nxt;
    }
}

// Dot products of the item in slot s into acc[row][position].
template <int M>
__device__ __forceinline__ void consume(const Slot &s, const ItemCur &c, const ActLds &A, float (&acc)[2][M]) {
    const int jl = threadIdx.x & 7;
    const int64_t nsub = c.K >> 5;
    const int it = c.item - (c.item >= c.s.nh ? c.s.nh : 0);
    if (c.qtype == SV_Q4_K) {
        const int t = c.s.w0 + it * 2;
        if (t < c.s.w1) step_terms<SV_Q4_K, 0, M>(s, A, t * 8 + jl - A.begin, acc, 0u, 0u);
        if (t + 1 < c.s.w1) step_terms<SV_Q4_K, 2, M>(s, A, (t + 1) * 8 + jl - A.begin, acc, 0u, 0u);
    } else {
        const int t = c.s.w0 + it;
        const int64_t sb = static_cast<int64_t>(t) * 8 + jl;
        if (t < c.s.w1 && sb < nsub) {
            const int sl = static_cast<int>(sb) - A.begin;
            if (c.qtype == SV_Q6_K) step_terms<SV_Q6_K, 0, M>(s, A, sl, acc, c.hs[0], c.hs[1]);
            else step_terms<SV_Q8_0, 0, M>(s, A, sl, acc, c.hs[0], c.hs[1]);
        }
    }
}

// End of a unit: the fixed-order sum of each row group's 8 lanes, written
// to the wave's partial slots [wave][matrix][position][row of the half
// tile] (matrix 1: the up half of a fused pair).
template <int M>
__device__ __forceinline__ void put_partials(float *wp, float (&acc)[2][M], int mm) {
    const int lane = threadIdx.x & 63;
    const int wave = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    const int grp = lane >> 3, jl = lane & 7;
    // every sum first (independent chains that fill each other's data-
    // parallel-move wait states), then the stores under one lane mask
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[p][m] = group8_sum(acc[p][m]);
    if (jl == 0) {
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
            for (int m = 0; m < M; m++) wp[((wave * NMat<M>::value + mm) * M + m) * 16 + grp * 2 + p] = acc[p][m];
    }
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[p][m] = 0.0f;
}

// State of a compute wave between ring items.
template <int M>
struct CompState {
    ItemCur L, C;     // load cursor (a ring ahead) and compute cursor
    bool lv, go;      // load cursor not yet past the end; compute cursor valid and no abort
    int buf;          // wave-partial buffer of the current unit
    int stb, stc;     // staged sub-blocks [stb, stb + stc) (as the control wave published them)
    ActLds A;
    float acc[2][M];  // the matrix being computed (gate, then up, of a fused pair)
    uint32_t lead;    // 1 in the younger wave of a SIMD: it leads a unit's items 0-1, 4-5, ...
};

// One ring step: consume the item in slot s (if the compute cursor is
// still valid), refill s with the item the load cursor points at, and close
// the unit if this was its last item.  The refill is issued on every step:
// a load cursor past the workgroup's last item reads that item again, so
// the loads in flight never depend on the path taken.
template <int M, class Tab>
__device__ __forceinline__ void ring_step(const Tab &tab, int n_phases, uint32_t b, uint32_t G, int wave,
                                          uint8_t *smem, Shared<M> &sh, CompState<M> &st, Slot &s) {
    // B1 opens a unit that starts a phase or whose K range lies outside
    // the staged one (the control wave takes the same decision)
    if (st.go && st.C.item == 0 &&
        (st.C.newphase || st.C.g.s_begin < st.stb || st.C.g.s_begin + st.C.g.cs > st.stb + st.stc)) {
        lds_barrier();   // B1: the unit's input is staged
        if (sh.abort) {
            st.go = false;
        } else {
            st.stb = sh.stb;
            st.stc = sh.stc;
            st.A = act_lds<M>(act_base<M>(smem), st.stc, st.stb);
        }
    }
    if (st.go) {
        // The two compute waves of a SIMD take the lead in turns, two items
        // each, the younger first.  At equal priority issue goes to the
        // older wave, which then runs ahead and leaves the younger one to
        // finish the unit alone, its latencies uncovered.
        if (((static_cast<uint32_t>(st.C.item) >> 1) + st.lead) & 1u) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        consume<M>(s, st.C, st.A, st.acc);
    }
    load_item(s, st.L);
    if (st.lv) st.lv = cur_advance_keep(tab, n_phases, b, G, st.L, wave, true);
    // a fused pair's gate sums are written after its last gate item
    if (st.go && st.C.fused && st.C.item == st.C.s.nh - 1) put_partials<M>(wpart_buf<M>(smem, st.buf), st.acc, 0);
    if (st.go && st.C.item == st.C.s.nitems - 1) {
        put_partials<M>(wpart_buf<M>(smem, st.buf), st.acc, st.C.fused ? 1 : 0);
        lds_barrier();   // B2: the unit's partial sums are written
        st.buf ^= 1;
        if (sh.abort) st.go = false;
    }
    if (st.go) st.go = cur_advance(tab, n_phases, b, G, st.C, wave, false);
}

template <int M, class Tab>
__device__ __forceinline__ void prime(const Tab &tab, int n_phases, uint32_t b, uint32_t G, int wave,
                                      CompState<M> &st, Slot &s) {
    load_item(s, st.L);
    if (st.lv) st.lv = cur_advance_keep(tab, n_phases, b, G, st.L, wave, true);
}

template <int M, class Tab>
__device__ __forceinline__ void compute_waves(const Tab &tab, int n_phases, uint32_t b, uint32_t G, uint8_t *smem,
                                              Shared<M> &sh) {
    constexpr int D = RingDepth<M>::value;
    const int wave = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    CompState<M> st;
    st.lead = wave >= kCompWaves / 2 ? 1u : 0u;   // waves w and w + 4 share a SIMD
    st.lv = cur_init(tab, n_phases, b, G, st.L, wave, true);
    st.go = cur_init(tab, n_phases, b, G, st.C, wave, false);
    if (!st.go) return;
    st.buf = 0;
    st.stb = 0;
    st.stc = -1;
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
        for (int m = 0; m < M; m++) st.acc[p][m] = 0.0f;
    // separate slots (no array): every access has a constant address from
    // the start, so the slots live in registers
    Slot s0, s1, s2, s3, s4, s5;
    prime<M>(tab, n_phases, b, G, wave, st, s0);
    prime<M>(tab, n_phases, b, G, wave, st, s1);
    if constexpr (D > 2) prime<M>(tab, n_phases, b, G, wave, st, s2);
    if constexpr (D > 3) prime<M>(tab, n_phases, b, G, wave, st, s3);
    if constexpr (D > 4) prime<M>(tab, n_phases, b, G, wave, st, s4);
    if constexpr (D > 5) prime<M>(tab, n_phases, b, G, wave, st, s5);
    while (st.go) {
        ring_step<M>(tab, n_phases, b, G, wave, smem, sh, st, s0);
        ring_step<M>(tab, n_phases, b, G, wave, smem, sh, st, s1);
        if constexpr (D > 2) ring_step<M>(tab, n_phases, b, G, wave, smem, sh, st, s2);
        if constexpr (D > 3) ring_step<M>(tab, n_phases, b, G, wave, smem, sh, st, s3);
        if constexpr (D > 4) ring_step<M>(tab, n_phases, b, G, wave, smem, sh, st, s4);
        if constexpr (D > 5) ring_step<M>(tab, n_phases, b, G, wave, smem, sh, st, s5);
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// ============================================================ control wave
__device__ __forceinline__ bool wait_ready(const unsigned *ctr, unsigned target, unsigned *status) {
    const int lane = threadIdx.x & 63;
    unsigned n = 0;
    // two polls in flight: the next read is issued before the previous one
    // is examined, so an update is seen about half a round trip sooner
    // every lane reads (lanes >= kSlots repeat the first slots), so no
    // branch hides the loads from the wait-count bookkeeping
    const int rep = static_cast<int>(blockIdx.x % kReplicas);
    const unsigned *slot = ctr + (rep * kSlots + (lane & (kSlots - 1))) * kSlotStride;
    unsigned a = ld_dev(slot);
    for (;;) {
        __builtin_amdgcn_s_sleep(2);
        const unsigned bb = ld_dev(slot);
        // the kSlots = 8 slots in lanes 0-7, added in lane 0 by data-parallel
        // moves (no LDS round trip), then read as a scalar
        static_assert(kSlots == 8, "the poll adds one group of eight lanes");
        int t = (lane < kSlots) ? static_cast<int>(a) : 0;
        t += dpp_i<0xB1>(t);    // quad_perm [1,0,3,2]
        t += dpp_i<0x4E>(t);    // quad_perm [2,3,0,1]
        t += dpp_i<0x104>(t);   // row_shl:4
        const unsigned v = static_cast<unsigned>(__builtin_amdgcn_readlane(t, 0));
        if (v >= target) return true;
        if (++n > kSpinLimit || ((n & 63u) == 0u && ld_dev(status) != 0u)) {
            if (lane == 0) or_dev(status, 1u);
            return false;
        }
        a = bb;
    }
}

// Copies n bytes (a multiple of 4) from global memory to LDS with the
// loads' LDS transfer: 16 bytes per lane when the source, the destination
// and the size allow it, else 4.  Lane l of an instruction writes dst + 16 l
// (or 4 l), so the LDS destination of each instruction is uniform.  The
// loops stay rolled: this code runs once per staged chunk, after a wait, so
// its length (instruction-cache misses), not its loop overhead, is what
// costs.  Whole-wave transfers run in a loop with a uniform trip count (no
// per-lane masking inside it), then one partial transfer takes the rest.
__device__ __forceinline__ void dma_copy(uint8_t *dst, const uint8_t *src, int n) {
    const uint32_t lane = threadIdx.x & 63;
    // size and both bases are wave-uniform: scalar loop control, and the
    // LDS address goes to M0 without a lane read each time
    const int nu = __builtin_amdgcn_readfirstlane(n);
    const uint32_t d0 = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>((uint32_t)(uintptr_t)(SV_AS3 uint8_t *)dst)));
    // readfirstlane returns a signed int: each half goes through uint32_t
    // before it is widened, so the low half is not sign-extended
    const uint64_t sa = reinterpret_cast<uint64_t>(src);
    const uint32_t slo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sa & 0xFFFFFFFFu)));
    const uint32_t shi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sa >> 32)));
    const uint64_t s0 = static_cast<uint64_t>(slo) | (static_cast<uint64_t>(shi) << 32);
    if (((s0 | d0 | static_cast<uint64_t>(nu)) & 15) == 0) {
        const int full = nu >> 10;                 // 1 KiB per whole-wave 16-byte transfer
        const int rest = (nu >> 4) - (full << 6);  // 16-byte pieces after them
        const uint64_t sl = s0 + lane * 16u;
#pragma unroll 1
        for (int k = 0; k < full; k++)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(sl + (static_cast<uint64_t>(k) << 10)),
                                             (SV_AS3 void *)static_cast<uintptr_t>(d0 + (k << 10)), 16, 0, 0);
        if (rest > 0 && static_cast<int>(lane) < rest)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(sl + (static_cast<uint64_t>(full) << 10)),
                                             (SV_AS3 void *)static_cast<uintptr_t>(d0 + (full << 10)), 16, 0, 0);
    } else {
        const int full = nu >> 8;                  // 256 bytes per whole-wave 4-byte transfer
        const int rest = (nu >> 2) - (full << 6);
        const uint64_t sl = s0 + lane * 4u;
#pragma unroll 1
        for (int k = 0; k < full; k++)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(sl + (static_cast<uint64_t>(k) << 8)),
                                             (SV_AS3 void *)static_cast<uintptr_t>(d0 + (k << 8)), 4, 0, 0);
        if (rest > 0 && static_cast<int>(lane) < rest)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(sl + (static_cast<uint64_t>(full) << 8)),
                                             (SV_AS3 void *)static_cast<uintptr_t>(d0 + (full << 8)), 4, 0, 0);
    }
}

// Copies M rows of `row` bytes, row m from src + m * sstride, into LDS rows
// LROW bytes apart (dst + m * LROW), in one loop over the LDS span
// (M - 1) LROW + row with 16-byte transfers; the caller checks that the
// addresses, the stride and the row are multiples of 16.  A lane whose piece
// falls in the tail of an LDS row, past its `row` bytes, loads the first
// piece of the field again (a valid address) into that tail, which nothing
// reads.  One loop instead of one copy per row: the per-copy set-up and the
// partial transfer that ends every copy are paid once.
template <int LROW>
__device__ __forceinline__ void dma_rows(uint8_t *dst, const uint8_t *src, int sstride, int row, int M) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t rowu = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(row));
    const uint32_t ssu = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(sstride));
    const int span = __builtin_amdgcn_readfirstlane((M - 1) * LROW + row);
    const uint32_t d0 = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>((uint32_t)(uintptr_t)(SV_AS3 uint8_t *)dst)));
    const uint64_t sa = reinterpret_cast<uint64_t>(src);
    const uint32_t slo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sa & 0xFFFFFFFFu)));
    const uint32_t shi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sa >> 32)));
    const uint64_t s0 = static_cast<uint64_t>(slo) | (static_cast<uint64_t>(shi) << 32);
    const int full = span >> 10;                 // 1 KiB per whole-wave transfer
    const int rest = (span >> 4) - (full << 6);  // 16-byte pieces after them
    uint32_t o = lane * 16u;                     // the lane's LDS offset in the span
#pragma unroll 1
    for (int k = 0; k < full; k++) {
        const uint32_t m = o / LROW, off = o - m * LROW;
        const uint64_t a = s0 + (off < rowu ? m * ssu + off : 0u);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(a),
                                         (SV_AS3 void *)static_cast<uintptr_t>(d0 + (k << 10)), 16, 0, 0);
        o += 1024u;
    }
    if (rest > 0 && static_cast<int>(lane) < rest) {
        const uint32_t m = o / LROW, off = o - m * LROW;
        const uint64_t a = s0 + (off < rowu ? m * ssu + off : 0u);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(a),
                                         (SV_AS3 void *)static_cast<uintptr_t>(d0 + (full << 10)), 16, 0, 0);
    }
}

// One field of the staged chunk: M rows of cs records of REC bytes, row m
// of the source at src + m * sstride, into LDS rows row_sub records apart.
template <int M, int REC>
__device__ __forceinline__ void stage_field(uint8_t *dst, const uint8_t *src, int sstride, int cs) {
    const int row = cs * REC, lrow = row_sub<M>(cs) * REC;
    if (sstride == row && row == lrow) {
        // the chunk is the whole row and fills the LDS row: the M rows are
        // contiguous in both
        dma_copy(dst, src, M * row);
        return;
    }
    if constexpr (M > 1) {
        const uint64_t al = reinterpret_cast<uint64_t>(src) | static_cast<uint64_t>(sstride) |
                            static_cast<uint64_t>(row) | static_cast<uint64_t>((uint32_t)(uintptr_t)(SV_AS3 uint8_t *)dst);
        if ((__builtin_amdgcn_readfirstlane(static_cast<int>(al & 15u))) == 0) {
            dma_rows<kRowSub * REC>(dst, src, sstride, row, M);
            return;
        }
    }
#pragma unroll 1
    for (int m = 0; m < M; m++) dma_copy(dst + m * lrow, src + static_cast<int64_t>(m) * sstride, row);
}

// The phase fields that staging and the RMS factors read, taken from the
// phase table before the wait for the input: the table is read through
// vector loads, and one issued after the wait would put a memory round trip
// in front of the staging transfers.
struct StageIn {
    const int8_t *aq;
    const float *ad;
    const int32_t *as16;
    const float *parts;
    int K, n_parts, parts_lds;
    float eps;
};
template <class PD>
__device__ __forceinline__ StageIn stage_in(const PD &P) {
    StageIn s;
    s.aq = P.aq;
    s.ad = P.ad;
    s.as16 = P.as16;
    s.parts = P.in_parts;
    s.K = P.K;
    s.n_parts = P.n_parts;
    s.parts_lds = P.parts_lds;
    s.eps = P.eps;
    return s;
}

// Copies the input chunk of a phase (codes, scales and code sums of every
// position and, where they fit the launch's LDS, the input's RMS partials)
// into LDS with load-to-LDS transfers and waits for them to land.
template <int M>
__device__ __forceinline__ void stage(const StageIn &P, const UnitPos &g, uint8_t *act, Shared<M> &sh,
                                      unsigned long long *tr) {
    const int lane = threadIdx.x & 63;
    const int K = P.K, nsub = K >> 5, cs = g.pcs, sb = g.pb;
    // the unit's chunk of S (which holds the unit's own range); three
    // fields, each M rows: codes (row stride K), scales (nsub floats),
    // code sums (K / 16 ints); in LDS each field's rows are row_sub records
    // apart, field after field
    const int rs = row_sub<M>(cs);
    stage_field<M, 32>(act, reinterpret_cast<const uint8_t *>(P.aq) + static_cast<int64_t>(sb) * 32, K, cs);
    stage_field<M, 4>(act + M * rs * 32, reinterpret_cast<const uint8_t *>(P.ad + sb), nsub * 4, cs);
    stage_field<M, 8>(act + M * rs * 36, reinterpret_cast<const uint8_t *>(P.as16 + 2 * sb), (K >> 4) * 4, cs);
    if (tr && lane == 0) tr[12] = now();
    // the transfers have written LDS once this wave's loads are complete
    __builtin_amdgcn_s_waitcnt(0);
    if (tr && lane == 0) tr[13] = now();
}

// The RMS factors of the staged input (only the control wave reads them, in
// the unit's finish, so they are formed after the compute waves are let go):
// lane l adds partials l, l + 64, ... in order, then wave_sum (a fixed order
// that depends only on the number of partials).  The partials come from LDS
// where they were staged, else from global memory, a position's loads all
// issued before the first add.
template <int M>
__device__ __forceinline__ void stage_rscale(const StageIn &P, const UnitPos &g, const uint8_t *act, Shared<M> &sh) {
    const int lane = threadIdx.x & 63;
    const int K = P.K, n_parts = P.n_parts;
    if (!P.parts) {
        if (lane < M) sh.rscale[lane] = 1.0f;
        return;
    }
    const float *lp = reinterpret_cast<const float *>(act + M * row_sub<M>(g.pcs) * kActRec);
    if (P.parts_lds) {
        // every position's partials of a lane at once (the positions'
        // reads and lane sums overlap); each position's adds keep their order
        float t[M];
#pragma unroll
        for (int m = 0; m < M; m++) t[m] = 0.0f;
        for (int i = lane; i < n_parts; i += 64)
#pragma unroll
            for (int m = 0; m < M; m++) t[m] += lp[m * n_parts + i];
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float tot = wave_sum(t[m]);
            if (lane == 0) sh.rscale[m] = 1.0f / sqrtf(tot / static_cast<float>(K) + P.eps);
        }
        return;
    }
#pragma unroll 1
    for (int m = 0; m < M; m++) {
        float t = 0.0f;
        {
            const float *gp = P.parts + m * n_parts;
            float v[kPartsPerLane];
#pragma unroll
            for (int k = 0; k < kPartsPerLane; k++) {
                const int i = lane + 64 * k;
                v[k] = i < n_parts ? gld(gp + i) : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kPartsPerLane; k++) t += v[k];
        }
        const float tot = wave_sum(t);
        if (lane == 0) sh.rscale[m] = 1.0f / sqrtf(tot / static_cast<float>(K) + P.eps);
    }
}

// Adds the workgroup's best (logit, index) keys of the phase to its argmax
// words.  In a pass those words are cleared by workgroup 0 at launch, so the
// control wave waits for the flag that says so (set within microseconds of
// the start, long before any head tile is done; bounded like every wait)
// before its first atomic maximum.
template <int M>
__device__ __forceinline__ void flush_best(unsigned long long *argmax, Shared<M> &sh, const unsigned *cleared,
                                           unsigned *status) {
    const int lane = threadIdx.x & 63;
    if (!argmax) return;
    if (cleared) {
        unsigned n = 0;
        while (ld_dev(cleared) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++n > kSpinLimit) {
                if (lane == 0) or_dev(status, 2u);
                break;
            }
        }
    }
    if (lane < M) {
        const unsigned long long v = sh.best[lane];
        if (v) max_dev(argmax + lane, v);
        sh.best[lane] = 0ull;
    }
}

// Values of a finished row tile in the control wave: lane l holds row
// r = l & 31 at positions m = (l >> 5) + 2k.
template <int M>
struct TileVals {
    float v[(M + 1) / 2];
};

template <int M, class PD>
__device__ __forceinline__ void store_y(const PD &P, int mt, int64_t row0, const TileVals<M> &x) {
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    const int64_t N = P.N;
    // integer arithmetic, not an index: an indexed pick from the three
    // fields would put them in memory
    const uint64_t m0 = mt == 0, m1 = mt == 1, m2 = mt == 2;
    float *y = reinterpret_cast<float *>(m0 * reinterpret_cast<uint64_t>(P.y[0]) +
                                         m1 * reinterpret_cast<uint64_t>(P.y[1]) +
                                         m2 * reinterpret_cast<uint64_t>(P.y[2]));
    if (!y) return;
    const int rows_here = static_cast<int>(min(static_cast<int64_t>(kRows), N - row0));
#pragma unroll
    for (int k = 0; k < (M + 1) / 2; k++) {
        const int m = h + 2 * k;
        if (m < M && r < rows_here) gst(y + static_cast<int64_t>(m) * N + row0 + r, x.v[k]);
    }
}

// Argmax candidates (the head's values x) and the requantised next
// activation from e (the epilogue's source: y[ep_src], or g*u for a pair):
// amax, d, codes, 16-element code sums and the sum of squares of each
// 32-row block, i.e. of one activation block.
template <int M, class PD>
__device__ __forceinline__ void finish_tile(const PD &P, int64_t row0, const TileVals<M> &x, const TileVals<M> &e,
                                            bool do_ep, float g_row, Shared<M> &sh) {
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    const int64_t N = P.N;
    const int rows_here = static_cast<int>(min(static_cast<int64_t>(kRows), N - row0));
    // The lane reductions that end in a cross-half permute through LDS are
    // formed for every position pair before any result is stored, so the
    // pairs' round trips overlap instead of running one after another
    // between the stores' branches.  Each pair's arithmetic is the same as
    // alone.
    constexpr int KP = (M + 1) / 2;
    unsigned long long *am = P.argmax;
    if (am) {
        unsigned long long bk[KP];
#pragma unroll
        for (int k = 0; k < KP; k++) {
            const unsigned long long key =
                r < rows_here ? pack_argmax(x.v[k], static_cast<uint32_t>(row0 + r)) : 0ull;
            bk[k] = half_max64(key);
        }
#pragma unroll
        for (int k = 0; k < KP; k++) {
            const int m = h + 2 * k;
            if (m < M && r == 0 && bk[k] > sh.best[m]) sh.best[m] = bk[k];
        }
    }
    if (do_ep && P.ep_mode != SV_EP_NONE && rows_here == kRows) {
        const float *gamma = P.gamma;
        int8_t *oq = P.oq;
        float *od = P.od, *osumsq = P.osumsq;
        int32_t *os16 = P.os16;
        const int64_t gb = row0 >> 5;
        float vg[KP], amx[KP], sq[KP];
#pragma unroll
        for (int k = 0; k < KP; k++) {
            const float v = e.v[k];
            vg[k] = gamma ? v * g_row : v;
            amx[k] = half_max(fabsf(vg[k]));
            sq[k] = half_sum(v * v);
        }
#pragma unroll
        for (int k = 0; k < KP; k++) {
            const int m = h + 2 * k;
            const float dd = amx[k] / 127.0f;
            const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
            float rq = roundf(vg[k] * id);
            rq = fminf(fmaxf(rq, -127.0f), 127.0f);
            const int qi = static_cast<int>(rq);
            const int sm = row_sum(qi);
            if (m < M) {
                st_dev(oq + m * N + row0 + r, static_cast<int8_t>(qi));
                if ((r & 15) == 0) st_dev(os16 + m * (N >> 4) + 2 * gb + (r >> 4), sm);
                if (r == 0) {
                    st_dev(od + m * (N >> 5) + gb, dd);
                    st_dev(osumsq + m * (N >> 5) + gb, sq[k]);
                }
            }
        }
    }
}

// The norm weight of the epilogue for row lane & 31 of unit u's tile,
// requested before the unit's barrier so it has arrived when the epilogue
// runs (1 when there is none).
// The phase fields a unit's finish reads, taken from the phase table while
// the unit computes: the table is read through vector loads, and the
// barrier before the finish orders memory, so a field first read after it
// would put a memory round trip in front of the unit's stores.  The names
// are the phase descriptor's, so the finish helpers take either.
struct FinishIn {
    int32_t N, n_w, fused, mu, S1, ep_mode, ep_src, count_all;
    float *y[3];
    const float *gamma;
    int8_t *oq;
    float *od;
    int32_t *os16;
    float *osumsq;
    unsigned long long *argmax;
    float *partial;
    unsigned *tile_count;
    unsigned *ready;
};
template <class PD>
__device__ __forceinline__ FinishIn finish_in(const PD &P) {
    FinishIn f;
    f.N = P.N;
    f.n_w = P.n_w;
    f.fused = P.fused;
    f.mu = P.mu;
    f.S1 = P.S1;
    f.ep_mode = P.ep_mode;
    f.ep_src = P.ep_src;
    f.count_all = P.count_all;
    f.y[0] = P.y[0];
    f.y[1] = P.y[1];
    f.y[2] = P.y[2];
    f.gamma = P.gamma;
    f.oq = P.oq;
    f.od = P.od;
    f.os16 = P.os16;
    f.osumsq = P.osumsq;
    f.argmax = P.argmax;
    f.partial = P.partial;
    f.tile_count = P.tile_count;
    f.ready = P.ready;
    return f;
}

__device__ __forceinline__ float gamma_of(const FinishIn &P, const UnitPos &g) {
    const float *gamma = P.gamma;
    if (!gamma || P.ep_mode == SV_EP_NONE) return 1.0f;
    const int64_t row = static_cast<int64_t>(g.tile) * kRows + (threadIdx.x & 31);
    return row < P.N ? gld(gamma + row) : 1.0f;
}


// The control wave's part of a unit whose partial sums sit in wave-partial
// buffer wp, right after the unit's barrier, in two halves.  finish_issue
// adds the four step quarters of each row in order (for both matrices of a
// fused pair), then either writes the tile's outputs, or (K split over
// units, or a pair whose matrices sit in two units) stores the chunk's
// values.  finish_complete, for a split tile, counts the chunk in once those
// stores have landed and, in the tile's last unit to arrive, adds all
// chunks in chunk order and writes the outputs; then it hands the unit off
// if a later phase reads it.
template <int M, class PD>
__device__ __forceinline__ bool unit_split(const PD &P, const UnitPos &g) {
    return g.nch > 1 || (P.ep_mode == SV_EP_PAIR && !P.fused);
}

template <int M>
__device__ __forceinline__ void finish_issue(const FinishIn &P, const UnitPos &g, const float *wp, float g_row,
                                             Shared<M> &sh, unsigned long long *tr) {
    if (tr && (threadIdx.x & 63) == 0) tr[7] = now();
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5, hr = r >> 4, rr = r & 15;
    const int64_t row0 = static_cast<int64_t>(g.tile) * kRows;
    const int64_t N = P.N;
    const int nm = P.fused ? 2 : 1;
    // the step quarters of each row, added in order: waves hr, hr + 2, ...
    TileVals<M> v0, v1;
#pragma unroll
    for (int k = 0; k < (M + 1) / 2; k++) {
        const int m = min(h + 2 * k, M - 1);
        constexpr int NM = NMat<M>::value;
        float a = wp[((hr * NM + 0) * M + m) * 16 + rr];
        float c = wp[((hr * NM + NM - 1) * M + m) * 16 + rr];
#pragma unroll
        for (int q = 1; q < kStepParts; q++) {
            a += wp[(((hr + 2 * q) * NM + 0) * M + m) * 16 + rr];
            c += wp[(((hr + 2 * q) * NM + NM - 1) * M + m) * 16 + rr];
        }
        v0.v[k] = a;
        v1.v[k] = c;
    }
    if (!unit_split<M>(P, g)) {
#pragma unroll
        for (int k = 0; k < (M + 1) / 2; k++) {
            const float rs = sh.rscale[min(h + 2 * k, M - 1)];
            v0.v[k] *= rs;
            v1.v[k] *= rs;
        }
        store_y<M>(P, g.mat, row0, v0);
        TileVals<M> e = v0;
        if (nm == 2) {
            store_y<M>(P, g.mat + 1, row0, v1);
#pragma unroll
            for (int k = 0; k < (M + 1) / 2; k++) e.v[k] = v0.v[k] * v1.v[k];
        }
        finish_tile<M>(P, row0, v0, e, nm == 2 || g.mat == P.ep_src, g_row, sh);
    } else {
        float *partial = P.partial;
        const int SP = P.S1;   // chunk slots per matrix
#pragma unroll
        for (int mm = 0; mm < 2; mm++) {
            if (mm < nm) {
#pragma unroll
                for (int k = 0; k < (M + 1) / 2; k++) {
                    const int m = h + 2 * k;
                    if (m < M && row0 + r < N)
                        st_dev(partial + ((static_cast<int64_t>(g.mat + mm) * SP + g.chunk) * M + m) * N + row0 + r,
                               mm ? v1.v[k] : v0.v[k]);
                }
            }
        }
    }
    if (tr && lane == 0) tr[8] = now();
}

template <int M>
__device__ __forceinline__ void finish_complete(const FinishIn &P, const UnitPos &g, uint32_t u, float g_row,
                                                Shared<M> &sh, unsigned long long *tr) {
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    const int64_t row0 = static_cast<int64_t>(g.tile) * kRows;
    const int64_t N = P.N;
    const bool pair = P.ep_mode == SV_EP_PAIR;
    if (unit_split<M>(P, g)) {
        float *partial = P.partial;
        const int SP = P.S1, S = g.nch;   // chunk slots per matrix; chunks of this tile
        drain();
        if (tr && lane == 0) tr[10] = now();
        unsigned *tc = P.tile_count;
        unsigned prev = 0;
        if (lane == 0) prev = add_dev(tc + g.tile, 1u);
        prev = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(prev), 0));
        if (prev == static_cast<unsigned>(S * P.mu - 1)) {
            const int n_w = P.n_w, src = P.ep_src;
            TileVals<M> f0, e;
#pragma unroll
            for (int mt = 0; mt < 3; mt++) {
                if (mt < n_w) {
                    TileVals<M> f;
                    // The partials of several position pairs are requested
                    // before any is used: one memory round trip for up to three
                    // pairs (M <= 6), one per two pairs up to M = 12 (more
                    // registers held here spill), one per pair above.  A row
                    // past N or a position past M reads an address that exists
                    // (row N - 1, position M - 1, chunk 0) and is dropped.
                    constexpr int KP = (M + 1) / 2, KG = KP <= 3 ? KP : 2;
                    if constexpr (M <= 12) {
                        const int64_t rc = min(row0 + r, N - 1);
#pragma unroll
                        for (int k0 = 0; k0 < KP; k0 += KG) {
                            float v[KG][kMaxS];
#pragma unroll
                            for (int kk = 0; kk < KG; kk++) {
                                const int mc = min(h + 2 * (k0 + kk), M - 1);
                                const float *srcp = partial + (static_cast<int64_t>(mt) * SP * M + mc) * N + rc;
#pragma unroll
                                for (int c = 0; c < kMaxS; c++)
                                    v[kk][c] = ld_dev(srcp + static_cast<int64_t>(c < S ? c : 0) * M * N);
                            }
#pragma unroll
                            for (int kk = 0; kk < KG && k0 + kk < KP; kk++) {
                                const int m = h + 2 * (k0 + kk);
                                float s = 0.0f;
                                if (m < M && row0 + r < N) {
#pragma unroll
                                    for (int c = 0; c < kMaxS; c++)
                                        if (c < S) s += v[kk][c];
                                }
                                f.v[k0 + kk] = s * sh.rscale[min(m, M - 1)];
                            }
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < KP; k++) {
                            const int m = h + 2 * k;
                            float s = 0.0f;
                            if (m < M && row0 + r < N) {
                                const float *srcp = partial + (static_cast<int64_t>(mt) * SP * M + m) * N + row0 + r;
                                float v[kMaxS];
#pragma unroll
                                for (int c = 0; c < kMaxS; c++) {
                                    // every chunk's partial is requested before any is used
                                    const float xx = ld_dev(srcp + static_cast<int64_t>(c < S ? c : 0) * M * N);
                                    v[c] = c < S ? xx : 0.0f;
                                }
#pragma unroll
                                for (int c = 0; c < kMaxS; c++)
                                    if (c < S) s += v[c];
                            }
                            f.v[k] = s * sh.rscale[min(m, M - 1)];
                        }
                    }
                    store_y<M>(P, mt, row0, f);
                    if (mt == 0) {
                        f0 = f;
                        e = f;
                    } else if (pair && mt == 1) {
#pragma unroll
                        for (int k = 0; k < (M + 1) / 2; k++) e.v[k] = f0.v[k] * f.v[k];
                    } else if (!pair && mt == src) {
                        e = f;
                    }
                }
            }
            if (lane == 0) st_dev(tc + g.tile, 0u);
            finish_tile<M>(P, row0, f0, e, true, g_row, sh);
        }
    }
    // hand-off: only units a later phase reads are counted
    unsigned *ready = P.ready;
    if (ready && (P.count_all || g.mat == P.ep_src)) {
        drain();
        if (tr && lane == 0) tr[11] = now();
        if (lane < kReplicas) add_dev(ready + (lane * kSlots + u % kSlots) * kSlotStride, 1u);
    }
}

template <int M, class Tab>
__device__ __forceinline__ void control_wave(const Tab &tab, int n_phases, uint32_t b, uint32_t G, uint8_t *smem,
                                             Shared<M> &sh, unsigned *status, const unsigned *cleared,
                                             unsigned long long *trace) {
    const int lane = threadIdx.x & 63;
    // The control wave issues first when it competes with the compute waves
    // for the SIMD and the memory pipeline: its few instructions (staging,
    // stores, hand-offs) are on the critical path of every phase, and it
    // sleeps while it waits, so it never starves them.
    __builtin_amdgcn_s_setprio(3);
    UnitCur c;
    unit_first(tab, n_phases, b, G, c);
    int pp = -1, buf = 0;
    // what is staged: the input codes, the chunk and the partials
    const int8_t *st_q = nullptr;
    const float *st_parts = nullptr;
    int st_begin = -1, st_cs = -1;
    unsigned long long *tr = nullptr;
    unsigned n_units = 0;
    uint8_t *act = act_base<M>(smem);
    while (c.p < n_phases) {
        const auto &P = tab[c.p];
        const UnitPos g = unit_pos(P, c.u);
        const bool phase_change = c.p != pp;
        // the unit's input is staged if it is the same input and its K range
        // lies inside the staged one (the compute waves test the range alone:
        // without a phase change the input is the same)
        const int8_t *aq = P.aq;
        const float *parts = P.in_parts;
        const bool inside = aq == st_q && parts == st_parts && g.s_begin >= st_begin &&
                            g.s_begin + g.cs <= st_begin + st_cs;
        if (phase_change || !(g.s_begin >= st_begin && g.s_begin + g.cs <= st_begin + st_cs)) {
            if (phase_change && pp >= 0) flush_best<M>(tab[pp].argmax, sh, cleared, status);
            if (phase_change) {
                if (tr && lane == 0) tr[6] = n_units;
                tr = trace ? trace + (static_cast<size_t>(b) * n_phases + c.p) * kTraceWords : nullptr;
                n_units = 0;
                if (tr && lane == 0) {
                    tr[0] = now();
                    tr[9] = static_cast<unsigned long long>(__builtin_amdgcn_s_getreg(0xF804)) |
                            (static_cast<unsigned long long>(__builtin_amdgcn_s_getreg(0xF814)) << 32);
                }
            }
            bool fresh = false;
            const StageIn si = stage_in(P);
            if (!inside) {
                const unsigned *wt = P.wait;
                if (wt && !wait_ready(wt, P.wait_target, status)) {
                    if (lane == 0) sh.abort = 1u;
                } else {
                    if (tr && lane == 0) tr[1] = now();
                    stage<M>(si, g, act, sh, tr);
                    if (tr && lane == 0) tr[2] = now();
                    st_q = aq;
                    st_parts = parts;
                    st_begin = g.pb;
                    st_cs = g.pcs;
                    fresh = true;
                }
            }
            if (lane == 0) {
                sh.stb = st_begin;
                sh.stc = st_cs;
            }
            lds_barrier();   // B1
            if (sh.abort) break;
            if (fresh) {
                // the input's RMS partials feed only this wave's finish: they
                // are staged after the compute waves are let go, so their
                // transfers do not hold up the barrier
                if (si.parts && si.parts_lds) {
                    dma_copy(act + M * row_sub<M>(g.pcs) * kActRec, reinterpret_cast<const uint8_t *>(si.parts),
                             M * si.n_parts * 4);
                    __builtin_amdgcn_s_waitcnt(0);
                }
                stage_rscale<M>(si, g, act, sh);
            }
        }
        const FinishIn fi = finish_in(P);       // in flight while the unit computes
        const float g_cur = gamma_of(fi, g);
        lds_barrier();       // B2: the compute waves have written the unit's partial sums
        if (sh.abort) break;
        unsigned long long *tf = n_units == 0 ? tr : nullptr;
        if (tf && lane == 0) tr[3] = now();
        finish_issue<M>(fi, g, wpart_buf<M>(smem, buf), g_cur, sh, tf);
        finish_complete<M>(fi, g, c.u, g_cur, sh, tf);
        if (tr && lane == 0) {
            if (tf) tr[4] = now();
            tr[5] = now();
        }
        n_units++;
        pp = c.p;
        buf ^= 1;
        unit_next(tab, n_phases, b, G, c);
    }
    if (pp >= 0 && !sh.abort) {
        if (tr && lane == 0) tr[6] = n_units;
        flush_best<M>(tab[pp].argmax, sh, cleared, status);
    }
    drain();
}

// ============================================================ kernels
// One workgroup per unit of a single phase.
template <int M>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void phase_kernel(PhaseDesc P) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ Shared<M> sh;
    if (threadIdx.x < SV_MAX_M) sh.best[threadIdx.x] = 0ull;
    if (threadIdx.x == 0) sh.abort = 0u;
    __syncthreads();
    // P is the launch's only argument, so it starts the argument segment
    (void)P;
    const OneTab tab{reinterpret_cast<const SV_AS4 PhaseDesc *>(
        reinterpret_cast<uintptr_t>(__builtin_amdgcn_kernarg_segment_ptr()))};
    if (threadIdx.x < kCompWaves * 64) compute_waves<M>(tab, 1, blockIdx.x, gridDim.x, smem, sh);
    else control_wave<M>(tab, 1, blockIdx.x, gridDim.x, smem, sh, nullptr, nullptr, nullptr);
}

// ctl: control words (kCtl*), then per phase kPhaseCounters counters of
// finished units, kSlotStride words apart.  The last workgroup to exit
// adds the run's status to kCtlResult (an OR the host reads and clears) and
// returns every other word to zero (and, after an expired wait, the tile
// counters of split tiles), so the next run starts clean without a reset
// launch.
template <int M>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void pass_kernel(const PhaseDesc *__restrict__ table, int n_phases,
                                                        const uint32_t *__restrict__ sched, unsigned *ctl, int CS,
                                                        ArgmaxList am, unsigned long long *trace) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ Shared<M> sh;
    __shared__ int last;
    unsigned *status = ctl + kCtlStatus;
    const unsigned *cleared = ctl + kCtlArgmaxClear;
    if (threadIdx.x < SV_MAX_M) sh.best[threadIdx.x] = 0ull;
    if (threadIdx.x == 0) sh.abort = 0u;
    // Workgroup 0 clears every argmax of the pass, waits until the stores
    // are done and raises the flag flush_best waits on.
    if (blockIdx.x == 0 && am.n > 0) {
        for (int i = 0; i < am.n; i++)
            if (static_cast<int>(threadIdx.x) < am.M[i]) st_dev(am.p[i] + threadIdx.x, 0ull);
        drain();
        __syncthreads();
        if (threadIdx.x == 0) st_dev(ctl + kCtlArgmaxClear, 1u);
    }
    __syncthreads();
    const ManyTab<M == 1> tab{reinterpret_cast<const SV_AS4 PhaseDesc *>(reinterpret_cast<uintptr_t>(table)),
                      reinterpret_cast<const SV_AS4 uint32_t *>(reinterpret_cast<uintptr_t>(sched)), n_phases,
                      gridDim.x};
    if (threadIdx.x < kCompWaves * 64) compute_waves<M>(tab, n_phases, blockIdx.x, gridDim.x, smem, sh);
    else control_wave<M>(tab, n_phases, blockIdx.x, gridDim.x, smem, sh, status, cleared, trace);
    __syncthreads();
    if (threadIdx.x == 0) last = (add_dev(ctl + kCtlExited, 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    if (last) {
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
