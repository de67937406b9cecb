// matvec_launch.h - the phase descriptor and launch entry points shared by
// the host side of the projection (matvec.hip) and the per-M kernel
// instantiations (matvec_inst.hip, compiled once per M so the sixteen
// variants build in parallel).
#pragma once

#include "sv_internal.h"

namespace sv {

constexpr int kThreads = 576;          // eight compute waves and one control wave
constexpr int kRows = 32;              // rows per tile: 2 half tiles of 8 groups x 2 rows
constexpr int kActRec = 32 + 4 + 8;    // LDS bytes per position per staged sub-block (codes, scale, sums)
constexpr int kMaxChunkSteps = 20;     // most 256-element steps of K one unit covers
constexpr int kRowSub = kMaxChunkSteps * 8;   // LDS row of a staged field: the largest chunk, in sub-blocks
// Records from one position's row of a staged field to the next: kRowSub
// with several positions (a position's offset is then a constant of the
// instruction), the chunk itself with one (there is no second row).
template <int M>
__host__ __device__ constexpr int row_sub(int cs) { return M == 1 ? cs : kRowSub; }
inline int row_sub_of(int M, int cs) { return M == 1 ? cs : kRowSub; }
constexpr int kMaxS = 8;               // most K chunks of a tile (K <= 40960)
constexpr int kBalanceGrid = 256;      // workgroups a balanced phase is cut for (one per CU)
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kMaxGrid = 1024;         // most workgroups a pass launches
constexpr int kMaxArgmax = 4;          // most phases of one pass with an argmax
constexpr int kPartsPerLane = 9;       // >= 576 RMS partials / 64 lanes

// Control words of a pass (one 256-byte line, word index): the live status
// of the running launch, the count of exited workgroups, the flag workgroup
// 0 raises once every argmax buffer is cleared, and the status of the last
// completed run.  The completion counters follow, from word kSlotStride on.
constexpr int kCtlStatus = 1;
constexpr int kCtlExited = 2;
constexpr int kCtlArgmaxClear = 3;
constexpr int kCtlResult = 4;

// Completion of a phase is counted in kSlots counters kSlotStride words
// apart (unit u adds to slot u % kSlots), so finishing units do not all
// serialise on one address; a waiter sums the slots.  The slots are kept in
// kReplicas copies: a finishing unit adds to every copy (one instruction,
// one lane per copy) and a waiter polls the copy of its workgroup index, so
// each counter line serves a quarter of the polling.
constexpr int kSlots = 8;
constexpr int kSlotStride = 64;
constexpr int kReplicas = 4;
constexpr int kPhaseCounters = kSlots * kReplicas;   // counter lines per phase

// Trace record of a (workgroup, phase): real-time counter at phase entry,
// input ready, input staged, first unit computed, first unit done, last
// unit done; units run; the first unit's finish: entry, outputs written,
// partial sums drained (split tiles); HW_ID | XCC_ID << 32; the first
// unit's hand-off drained; the first staging's transfers issued, and
// landed; two unused.
constexpr int kTraceWords = 16;

// Division by a divisor d >= 1 fixed per phase: n / d = (n * m) >> sh for
// every n < 2^31, with l = ceil(log2 d), m = ceil(2^(31 + l) / d) and
// sh = 31 + l (the round-up method of Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994).  The unit geometry is
// derived with it from scalar registers, instead of the long vector
// sequence of a general integer division.
struct FastDiv {
    uint32_t m, sh;
};

// Device-side description of one phase.
struct PhaseDesc {
    const uint8_t *w[3];
    int32_t qtype, n_w, M;
    int32_t N, K, wrows;
    // K chunking: tiles [0, T1) are cut into S chunks, tiles [T1, n_tiles)
    // into S1 (a multiple of S); a unit covers mu matrices' worth of one
    // (tile, chunk): per_tile = S * mu units per tile of the first kind.
    int32_t S, S1, T1, mu, steps, n_tiles, per_tile, n_units, chunk_sub;
    FastDiv div_pt, div_S, div_f, div_S1;   // by per_tile, S, S1 / S and S1
    int32_t count_all;        // 0: only units of matrix ep_src feed a reader
    int32_t fused;            // 1: a unit covers both matrices of a gate/up pair (M <= 8)
    uint32_t bbytes;          // bytes of a weight block (16 rows x 256 columns)
    const int32_t *row_ids;
    const int8_t *aq;
    const float *ad;
    const int32_t *as16;
    const float *in_parts;
    int32_t n_parts;
    int32_t parts_lds;        // 1: the partials are staged into LDS after the chunk
    float eps;
    float *y[3];
    int32_t ep_mode, ep_src;
    const float *gamma;
    int8_t *oq;
    float *od;
    int32_t *os16;
    float *osumsq;
    unsigned long long *argmax;
    float *partial;           // [n_w][S1][M][N] when a tile is split over units
    unsigned *tile_count;     // [n_tiles], zero between calls
    unsigned *ready;          // finished units of this phase (persistent mode; NULL: no reader)
    const unsigned *wait;     // finished units of the input's producer (NULL: input written before)
    uint32_t wait_target;
};

// The argmax buffers a pass clears before any head workgroup adds to them.
struct ArgmaxList {
    unsigned long long *p[kMaxArgmax];
    int32_t M[kMaxArgmax];
    int32_t n;
};

// Defined once per M in matvec_inst.hip.
template <int M>
void launch_pass_m(int grid, size_t lds, hipStream_t st, const PhaseDesc *table, int n_phases, const uint32_t *sched,
                   unsigned *ctl, int CS, ArgmaxList am, unsigned long long *trace);
template <int M>
void launch_phase_m(int grid, size_t lds, hipStream_t st, const PhaseDesc &P, int CS);
template <int M>
int occupancy_pass_m(size_t lds);
template <int M>
hipError_t allow_lds_m(size_t lds);
template <int M>
hipError_t pass_attr_m(hipFuncAttributes *fa);

}  // namespace sv
