// matvec.hip - host side of the verification projection (a3/a4), the head
// (a6/a9) and the whole pass (a5): argument validation, the decomposition
// of a phase into units, scratch layout, the dependency graph of a pass and
// the launches.  The kernels are in matvec_dev.h, instantiated per M by
// matvec_inst.hip.
//
// A pass is a list of phases ("Inside OpenJet Engine: making speculative
// decoding pay", section "One GPU launch for a speculative cycle": the
// phases of a cycle in one launch, synchronised between phases).  A phase
// waits only for the phase that wrote its input: the producer is the latest
// earlier phase whose epilogue outputs are exactly the phase's input
// buffers, and a phase whose input no earlier phase writes starts at once.
// So phases that read the same input (q and k beside v, say) run side by
// side, and matrices of different formats on one input are simply separate
// phases.
#include <algorithm>
#include <array>
#include <utility>
#include <vector>

#include "matvec_launch.h"

namespace sv {

// ------------------------------------------------------------- dispatch
using PassFn = void (*)(int, size_t, hipStream_t, const PhaseDesc *, int, const uint32_t *, unsigned *, int, ArgmaxList,
                        unsigned long long *);
using PhaseFn = void (*)(int, size_t, hipStream_t, const PhaseDesc &, int);
using OccFn = int (*)(size_t);
using LdsFn = hipError_t (*)(size_t);
using AttrFn = hipError_t (*)(hipFuncAttributes *);

template <size_t... I>
static constexpr std::array<PassFn, SV_MAX_M> pass_fns(std::index_sequence<I...>) {
    return {&launch_pass_m<static_cast<int>(I) + 1>...};
}
template <size_t... I>
static constexpr std::array<PhaseFn, SV_MAX_M> phase_fns(std::index_sequence<I...>) {
    return {&launch_phase_m<static_cast<int>(I) + 1>...};
}
template <size_t... I>
static constexpr std::array<OccFn, SV_MAX_M> occ_fns(std::index_sequence<I...>) {
    return {&occupancy_pass_m<static_cast<int>(I) + 1>...};
}
template <size_t... I>
static constexpr std::array<LdsFn, SV_MAX_M> lds_fns(std::index_sequence<I...>) {
    return {&allow_lds_m<static_cast<int>(I) + 1>...};
}
static const std::array<PassFn, SV_MAX_M> kPassFns = pass_fns(std::make_index_sequence<SV_MAX_M>{});
static const std::array<PhaseFn, SV_MAX_M> kPhaseFns = phase_fns(std::make_index_sequence<SV_MAX_M>{});
static const std::array<OccFn, SV_MAX_M> kOccFns = occ_fns(std::make_index_sequence<SV_MAX_M>{});
template <size_t... I>
static constexpr std::array<AttrFn, SV_MAX_M> attr_fns(std::index_sequence<I...>) {
    return {&pass_attr_m<static_cast<int>(I) + 1>...};
}
static const std::array<LdsFn, SV_MAX_M> kLdsFns = lds_fns(std::make_index_sequence<SV_MAX_M>{});
static const std::array<AttrFn, SV_MAX_M> kAttrFns = attr_fns(std::make_index_sequence<SV_MAX_M>{});

// Workgroups of the pass kernel one compute unit holds at once, counted
// from what a workgroup takes: its waves against the SIMDs' wave slots and
// its LDS against the unit's.  A SIMD holds 512 / registers-per-wave waves
// (at most 8); the waves of a workgroup are spread over the four SIMDs, so
// one SIMD carries ceil(waves / 4) of every workgroup (a five-wave
// workgroup puts two on one SIMD, and two such workgroups cannot share a
// unit whose SIMDs hold three waves each: measured).  The smaller of this
// and the runtime's occupancy figure is used, so a grid never holds more
// workgroups than can be resident together (they wait on each other).
static int resident_per_cu(int M, size_t lds, const hipDeviceProp_t &prop, int occ_api) {
    hipFuncAttributes fa;
    if (kAttrFns[M - 1](&fa) != hipSuccess) return 0;
    const int regs = std::max(8, (fa.numRegs + 7) / 8 * 8);
    const int waves_simd = std::min(8, 512 / regs);
    const int waves_wg = (kThreads + 63) / 64;
    const int by_waves = waves_simd / ((waves_wg + 3) / 4);
    const size_t lds_cu = prop.maxSharedMemoryPerMultiProcessor ? prop.maxSharedMemoryPerMultiProcessor : 160 * 1024;
    const int by_lds = static_cast<int>(lds_cu / std::max<size_t>(1, lds + fa.sharedSizeBytes));
    return std::min(std::min(occ_api, by_waves), by_lds);
}

constexpr size_t kDefaultLds = 64 * 1024;
constexpr size_t kStaticLds = 1024;   // held for the kernels' own __shared__ variables (224 bytes today)

// Largest dynamic LDS one workgroup may use on the current device: the
// device's LDS per workgroup less what the kernels declare statically.
static int lds_limit(size_t *limit) {
    int dev = 0;
    hipDeviceProp_t prop;
    int rc = hip_check(hipGetDevice(&dev), "device query");
    if (!rc) rc = hip_check(hipGetDeviceProperties(&prop, dev), "device query");
    if (rc) return rc;
    *limit = std::max(static_cast<size_t>(prop.sharedMemPerBlock) - kStaticLds, kDefaultLds);
    return SV_OK;
}

// Checks the LDS size against the device and, above the default, allows it
// for the kernels of this M.
static int prepare_lds(int M, size_t lds) {
    if (lds <= kDefaultLds) return SV_OK;
    size_t limit = 0;
    int rc = lds_limit(&limit);
    if (rc) return rc;
    SV_REQUIRE(lds <= limit, SV_ERR_SHAPE,
               "the input chunk, row tile and RMS partials need " + std::to_string(lds) +
                   " bytes of LDS; the device allows " + std::to_string(limit));
    return hip_check(kLdsFns[M - 1](lds), "allow LDS");
}

// Decomposition of a phase.  K is cut into S = ceil(steps / 20) chunks.
// A balanced phase (every projection that is not a head) with at least a
// round of kBalanceGrid tile-chunks also cuts the tiles of its last partial
// round finer: the remainder R of tile-chunks over whole rounds is spread as
// S1 = f S chunks on the last ceil(R / S) tiles, so the phase fills whole
// rounds and no workgroup runs a full unit while the others wait.  The
// chunking is a function of K and the row count only (not of M, nor of the
// other matrices of the call), so the batch invariance of every row holds;
// a head keeps S chunks on every tile, so a restricted head scores a row
// exactly as the full head does.
static FastDiv fast_div(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) l++;
    const unsigned __int128 num = static_cast<unsigned __int128>(1) << (31 + l);
    return FastDiv{static_cast<uint32_t>((num + d - 1) / d), 31 + l};
}

static void decompose(PhaseDesc &P, bool balance) {
    const int64_t nsub = P.K / 32;
    P.steps = static_cast<int>((nsub + 7) / 8);
    P.S = std::max(1, (P.steps + kMaxChunkSteps - 1) / kMaxChunkSteps);
    P.n_tiles = static_cast<int>((static_cast<int64_t>(P.N) + kRows - 1) / kRows);
    P.S1 = P.S;
    P.T1 = P.n_tiles;
    const int64_t tc = static_cast<int64_t>(P.n_tiles) * P.S;
    if (balance && tc >= kBalanceGrid && tc % kBalanceGrid) {
        const int64_t R = tc % kBalanceGrid;
        const int tr = static_cast<int>((R + P.S - 1) / P.S);
        const int f = std::min({kBalanceGrid / (tr * P.S), kMaxS / P.S, P.steps / P.S});
        if (f >= 2) {
            P.T1 = P.n_tiles - tr;
            P.S1 = P.S * f;
        }
    }
    // For M <= 8 a unit of a gate/up pair covers both matrices; above that
    // each matrix is a unit of its own and the tile's last unit forms the
    // product.
    P.fused = (P.ep_mode == SV_EP_PAIR && P.n_w == 2 && P.M <= 8) ? 1 : 0;
    P.mu = P.fused ? 1 : P.n_w;
    P.per_tile = P.S * P.mu;
    P.n_units = P.T1 * P.per_tile + (P.n_tiles - P.T1) * P.S1 * P.mu;
    P.chunk_sub = ((P.steps + P.S - 1) / P.S) * 8;
    P.div_pt = fast_div(static_cast<uint32_t>(P.per_tile));
    P.div_S = fast_div(static_cast<uint32_t>(P.S));
    P.div_f = fast_div(static_cast<uint32_t>(P.S1 / P.S));
    P.div_S1 = fast_div(static_cast<uint32_t>(P.S1));
}

// LDS of a workgroup: the compute waves' partial sums (two buffers, two
// matrices each where a unit may cover a fused pair, M <= 8), then the
// staged input chunk of all M positions and, where P.parts_lds, the RMS
// partials of the input; the largest phase sets the size.
static size_t wpart_bytes(int M) { return static_cast<size_t>(2) * 8 * (M <= 8 ? 2 : 1) * M * 16 * 4; }

static size_t parts_bytes(const PhaseDesc &P, int M) {
    return P.in_parts ? static_cast<size_t>(M) * P.n_parts * 4 : 0;
}

static size_t phase_lds(const PhaseDesc &P, int M) {
    return static_cast<size_t>(M) * row_sub_of(M, P.chunk_sub) * kActRec + (P.parts_lds ? parts_bytes(P, M) : 0);
}

// Stages the RMS partials of a phase's input into LDS when the phase's LDS
// still fits the device with them (the factors are then formed from LDS
// right after the staging wait); otherwise that phase's factors read them
// from global memory.  The sum is the same either way.
static int place_parts(PhaseDesc *P, int n, int M) {
    size_t limit = 0;
    bool queried = false;
    for (int i = 0; i < n; i++) {
        const size_t with =
            static_cast<size_t>(M) * row_sub_of(M, P[i].chunk_sub) * kActRec + parts_bytes(P[i], M) + wpart_bytes(M);
        if (with > kDefaultLds && !queried) {
            const int rc = lds_limit(&limit);
            if (rc) return rc;
            queried = true;
        }
        P[i].parts_lds = P[i].in_parts && (with <= kDefaultLds || with <= limit) ? 1 : 0;
    }
    return SV_OK;
}

static bool needs_partials(const PhaseDesc &P) {
    return P.S1 > 1 || (P.ep_mode == SV_EP_PAIR && !P.fused);
}

static size_t partial_bytes(const PhaseDesc &P, int M) {
    if (!needs_partials(P)) return 0;
    return static_cast<size_t>(P.n_w) * P.S1 * M * static_cast<size_t>(P.N) * 4;
}

static size_t round256(size_t n) { return (n + 255) / 256 * 256; }

static int validate_act(const sv_act *A) {
    SV_REQUIRE(A, SV_ERR_ARG, "activation descriptor is NULL");
    SV_REQUIRE(A->M >= 1 && A->M <= SV_MAX_M, SV_ERR_ARG, "M must be in [1, 16]");
    SV_REQUIRE(A->q && A->d && A->s16, SV_ERR_ARG, "activation buffers must not be NULL");
    SV_REQUIRE(A->K > 0 && A->K % 32 == 0 && A->K <= kMaxS * kMaxChunkSteps * 256, SV_ERR_SHAPE,
               "activation K must be a positive multiple of 32, at most 40960");
    SV_REQUIRE(aligned(A->q, 16) && aligned(A->d, 4) && aligned(A->s16, 8), SV_ERR_ALIGN,
               "activation codes must be 16-byte aligned, scales 4-byte, sums 8-byte");
    if (A->sumsq_parts) {
        SV_REQUIRE(A->n_parts >= 1 && A->n_parts <= kPartsPerLane * 64, SV_ERR_ARG,
                   "n_parts must be in [1, 576] when sumsq_parts is given");
        SV_REQUIRE(aligned(A->sumsq_parts, 4), SV_ERR_ALIGN, "sumsq_parts must be 4-byte aligned");
    }
    return SV_OK;
}

static int validate_weight(const sv_weight &W, int64_t K) {
    SV_REQUIRE(W.data, SV_ERR_ARG, "weight data is NULL");
    SV_REQUIRE(W.qtype == SV_Q8_0 || W.qtype == SV_Q4_K || W.qtype == SV_Q6_K, SV_ERR_QTYPE,
               "unsupported qtype " + std::to_string(W.qtype));
    Blocked L;
    SV_REQUIRE(blocked_of(W.qtype, W.rows, W.cols, &L), SV_ERR_SHAPE,
               "weight cols must be a multiple of 32 (Q8_0) or 256 (Q4_K, Q6_K)");
    SV_REQUIRE(L.total - kTailPad < (static_cast<size_t>(1) << 32), SV_ERR_SHAPE,
               "a repacked matrix must stay under 4 GiB");
    SV_REQUIRE(W.cols == K, SV_ERR_SHAPE, "weight cols must equal the activation K");
    SV_REQUIRE(W.rows < (1ll << 31), SV_ERR_SHAPE, "weight rows must be < 2^31");
    SV_REQUIRE(aligned(W.data, 256), SV_ERR_ALIGN, "repacked weights must be 256-byte aligned");
    return SV_OK;
}

// Fill a PhaseDesc from ABI arguments (no scratch pointers yet).
static int make_phase(PhaseDesc &P, const sv_weight *W, int32_t n_w, const sv_act *A, float *const *y,
                      const sv_epilogue *ep, const int32_t *row_ids, int64_t n_rows, uint64_t *argmax,
                      bool balance) {
    SV_REQUIRE(W, SV_ERR_ARG, "weights are NULL");
    SV_REQUIRE(n_w >= 1 && n_w <= 3, SV_ERR_ARG, "n_w must be 1..3");
    int rc = validate_act(A);
    if (rc) return rc;
    for (int i = 0; i < n_w; i++) {
        rc = validate_weight(W[i], A->K);
        if (rc) return rc;
        SV_REQUIRE(W[i].qtype == W[0].qtype && W[i].rows == W[0].rows, SV_ERR_SHAPE,
                   "matrices sharing an input in one call must have the same qtype and rows "
                   "(in a pass, put matrices of another format on the same input in a phase of their own)");
    }
    if (row_ids) SV_REQUIRE(n_rows >= 1 && n_rows < (1ll << 31), SV_ERR_SHAPE, "n_rows out of range");
    P = PhaseDesc{};
    P.qtype = W[0].qtype;
    P.n_w = n_w;
    P.wrows = static_cast<int32_t>(W[0].rows);
    P.N = static_cast<int32_t>(row_ids ? n_rows : W[0].rows);
    P.K = static_cast<int32_t>(A->K);
    P.M = A->M;
    P.bbytes = block_bytes(W[0].qtype);
    for (int i = 0; i < n_w; i++) {
        P.w[i] = static_cast<const uint8_t *>(W[i].data);
        P.y[i] = y ? y[i] : nullptr;
        if (P.y[i]) SV_REQUIRE(aligned(P.y[i], 4), SV_ERR_ALIGN, "outputs must be 4-byte aligned");
    }
    P.row_ids = row_ids;
    P.aq = A->q;
    P.ad = A->d;
    P.as16 = A->s16;
    P.in_parts = A->sumsq_parts;
    P.n_parts = A->sumsq_parts ? A->n_parts : 0;
    P.eps = A->eps;
    P.argmax = reinterpret_cast<unsigned long long *>(argmax);
    if (argmax) SV_REQUIRE(aligned(argmax, 8), SV_ERR_ALIGN, "argmax must be 8-byte aligned");
    P.ep_mode = SV_EP_NONE;
    if (ep && ep->mode != SV_EP_NONE) {
        SV_REQUIRE(ep->mode == SV_EP_QUANT || ep->mode == SV_EP_PAIR, SV_ERR_ARG, "bad epilogue mode");
        SV_REQUIRE(P.N % 32 == 0, SV_ERR_SHAPE, "the epilogue needs rows % 32 == 0");
        SV_REQUIRE(ep->q && ep->d && ep->s16 && ep->sumsq, SV_ERR_ARG, "epilogue outputs are NULL");
        SV_REQUIRE(aligned(ep->q, 16) && aligned(ep->d, 4) && aligned(ep->s16, 8) && aligned(ep->sumsq, 4) &&
                       (!ep->gamma || aligned(ep->gamma, 4)),
                   SV_ERR_ALIGN, "epilogue buffer alignment");
        if (ep->mode == SV_EP_QUANT)
            SV_REQUIRE(ep->src >= 0 && ep->src < n_w, SV_ERR_ARG, "epilogue src out of range");
        else
            SV_REQUIRE(n_w == 2, SV_ERR_ARG, "the pair epilogue needs exactly two matrices");
        P.ep_mode = ep->mode;
        P.ep_src = ep->src;
        P.gamma = ep->gamma;
        P.oq = ep->q;
        P.od = ep->d;
        P.os16 = ep->s16;
        P.osumsq = ep->sumsq;
    }
    decompose(P, balance);
    return SV_OK;
}

// Scratch of a single call: a fixed counter region (the same for every
// call, so a workspace shared by calls of different shapes never has
// partial sums where another call keeps its counters) followed by the
// partial sums.
constexpr size_t kCounterBytes = 256 * 1024;
constexpr int kMaxTiles = static_cast<int>(kCounterBytes / 4);

static size_t phase_scratch(const PhaseDesc &P, int M) {
    if (!needs_partials(P)) return 0;
    return kCounterBytes + partial_bytes(P, M);
}

static int launch_single(PhaseDesc &P, int M, void *ws, size_t ws_bytes, hipStream_t st) {
    const size_t need = phase_scratch(P, M);
    if (needs_partials(P)) {
        SV_REQUIRE(ws && ws_bytes >= need, SV_ERR_WORKSPACE,
                   "workspace needs " + std::to_string(need) + " bytes");
        SV_REQUIRE(aligned(ws, 256), SV_ERR_ALIGN, "workspace must be 256-byte aligned");
        SV_REQUIRE(P.n_tiles <= kMaxTiles, SV_ERR_SHAPE, "too many row tiles for the counter region");
        uint8_t *b = static_cast<uint8_t *>(ws);
        P.tile_count = reinterpret_cast<unsigned *>(b);
        P.partial = reinterpret_cast<float *>(b + kCounterBytes);
    }
    const int CS = P.chunk_sub;
    int rc = place_parts(&P, 1, M);
    if (rc) return rc;
    const size_t lds = wpart_bytes(M) + phase_lds(P, M);
    rc = prepare_lds(M, lds);
    if (rc) return rc;
    kPhaseFns[M - 1](P.n_units, lds, st, P, CS);
    return hip_check(hipGetLastError(), "projection launch");
}

__global__ void zero_u64(unsigned long long *p, int n) {
    if (static_cast<int>(threadIdx.x) < n) p[threadIdx.x] = 0ull;
}

}  // namespace sv

// ----------------------------------------------------------------- ABI
extern "C" size_t sv_matvec_workspace_bytes(const sv_weight *W, int32_t n_w, const sv_act *A) {
    sv::PhaseDesc P;
    if (sv::make_phase(P, W, n_w, A, nullptr, nullptr, nullptr, 0, nullptr, true) != SV_OK) return 0;
    // sized for any epilogue: two matrices may be paired
    if (n_w == 2) {
        P.ep_mode = SV_EP_PAIR;
        sv::decompose(P, true);
    }
    return sv::phase_scratch(P, A->M);
}

extern "C" int sv_verify_matvec(const sv_weight *W, int32_t n_w, const sv_act *A, float *const *y,
                                const sv_epilogue *ep, void *workspace, size_t ws_bytes, void *stream) {
    sv::PhaseDesc P;
    int rc = sv::make_phase(P, W, n_w, A, y, ep, nullptr, 0, nullptr, true);
    if (rc) return rc;
    return sv::launch_single(P, A->M, workspace, ws_bytes, sv::as_stream(stream));
}

extern "C" size_t sv_head_workspace_bytes(const sv_weight *H, const sv_act *A, int64_t n_rows) {
    sv::PhaseDesc P;
    if (sv::make_phase(P, H, 1, A, nullptr, nullptr, nullptr, 0, nullptr, false) != SV_OK) return 0;
    if (n_rows > 0) {
        P.N = static_cast<int32_t>(n_rows);
        sv::decompose(P, false);
    }
    return sv::phase_scratch(P, A->M);
}

extern "C" int sv_head_logits(const sv_weight *H, const sv_act *A, const int32_t *row_ids, int64_t n_rows,
                              float *logits, uint64_t *argmax, void *workspace, size_t ws_bytes, void *stream) {
    using namespace sv;
    SV_REQUIRE(H, SV_ERR_ARG, "head_logits: H is NULL");
    if (!row_ids) n_rows = H->rows;
    SV_REQUIRE(n_rows >= 1 && n_rows < (1ll << 31), SV_ERR_SHAPE, "head_logits: n_rows out of range");
    SV_REQUIRE(logits || argmax, SV_ERR_ARG, "head_logits: nothing to write");
    SV_REQUIRE(!logits || aligned(logits, 4), SV_ERR_ALIGN, "head_logits: logits must be 4-byte aligned");
    SV_REQUIRE(!argmax || aligned(argmax, 8), SV_ERR_ALIGN, "head_logits: argmax must be 8-byte aligned");
    SV_REQUIRE(!row_ids || aligned(row_ids, 4), SV_ERR_ALIGN, "head_logits: row_ids must be 4-byte aligned");
    float *ys[1] = {logits};
    PhaseDesc P;
    int rc = make_phase(P, H, 1, A, ys, nullptr, row_ids, n_rows, argmax, false);
    if (rc) return rc;
    hipStream_t st = as_stream(stream);
    if (argmax) {
        hipLaunchKernelGGL(zero_u64, dim3(1), dim3(64), 0, st, P.argmax, A->M);
        rc = hip_check(hipGetLastError(), "head_logits init");
        if (rc) return rc;
    }
    return launch_single(P, A->M, workspace, ws_bytes, st);
}

// ------------------------------------------------------------ whole pass
struct sv_pass {
    int M, n_phases, grid, CS, NP;
    size_t lds;
    sv::PhaseDesc *table;        // device
    uint32_t *sched;             // device: per-workgroup unit lists (see schedule)
    unsigned *ctl;               // device: control words, completion slots
    unsigned long long *trace;   // device: [kMaxGrid][n_phases][kTraceWords]
    sv::ArgmaxList am;
    bool tracing;
    std::vector<sv::PhaseDesc> host;
};

namespace sv {

// Workspace of a pass, in order: phase table | schedule | control words
// and completion counters | trace | per phase with split tiles: its tile
// counters, then its partial sums.  Every phase has scratch of its own, so
// phases that run side by side never share counters or partials.
struct PassLayout {
    size_t table, sched, ctl, trace, scratch, total;
    std::vector<size_t> tiles_off, part_off;   // per phase, from the start of the scratch
};

static int plan_pass(const sv_phase *phases, int32_t n_phases, std::vector<PhaseDesc> &host, PassLayout &L) {
    SV_REQUIRE(phases && n_phases >= 1, SV_ERR_ARG, "pass: no phases");
    host.assign(n_phases, PhaseDesc{});
    L.tiles_off.assign(n_phases, 0);
    L.part_off.assign(n_phases, 0);
    size_t scratch = 0;
    for (int i = 0; i < n_phases; i++) {
        const sv_phase &ph = phases[i];
        // a head phase (row gather or argmax) is cut as sv_head_logits cuts
        // it, every other phase as sv_verify_matvec does
        int rc = make_phase(host[i], ph.W, ph.n_w, &ph.A, ph.y, ph.ep.mode ? &ph.ep : nullptr, ph.row_ids, ph.n_rows,
                            ph.argmax, !(ph.row_ids || ph.argmax));
        if (rc) return fail(rc, "pass: phase " + std::to_string(i) + ": " + std::string(sv_last_error()));
        SV_REQUIRE(ph.A.M == phases[0].A.M, SV_ERR_SHAPE, "pass: all phases need the same M");
        if (needs_partials(host[i])) {
            L.tiles_off[i] = scratch;
            scratch += round256(static_cast<size_t>(host[i].n_tiles) * 4);
            L.part_off[i] = scratch;
            scratch += round256(partial_bytes(host[i], ph.A.M));
        }
    }
    size_t units = 0;
    for (const PhaseDesc &P : host) {
        SV_REQUIRE(P.n_units < (1 << 20), SV_ERR_SHAPE, "pass: a phase has more than 2^20 units");
        units += static_cast<size_t>(P.n_units);
    }
    SV_REQUIRE(n_phases < (1 << 12), SV_ERR_ARG, "pass: at most 4095 phases");
    L.table = round256(static_cast<size_t>(n_phases) * sizeof(PhaseDesc));
    L.sched = round256((static_cast<size_t>(kMaxGrid) + 1 + units) * 4);
    L.ctl = round256(static_cast<size_t>(kSlotStride) * (1 + n_phases * kPhaseCounters) * 4);
    L.trace = round256(static_cast<size_t>(kMaxGrid) * n_phases * kTraceWords * 8);
    L.scratch = scratch;
    L.total = L.table + L.sched + L.ctl + L.trace + L.scratch;
    return SV_OK;
}

// The unit geometry of the device's unit_pos, for the host's schedule.
static void host_unit_range(const PhaseDesc &P, uint32_t u, int &c0, int &c1, int &s_begin, int &cs, int &pb,
                            int &pcs) {
    const int per_tile = P.per_tile, S = P.S, head = P.T1 * per_tile;
    int chunk, nch, parent;
    if (static_cast<int>(u) < head) {
        chunk = (static_cast<int>(u) % per_tile) % S;
        nch = S;
        parent = chunk;
    } else {
        const int v = static_cast<int>(u) - head, f = P.S1 / S;
        const int rem = v % per_tile, q = v / per_tile;
        parent = rem % S;
        chunk = f * parent + q % f;
        nch = P.S1;
    }
    c0 = chunk * P.steps / nch;
    c1 = (chunk + 1) * P.steps / nch;
    s_begin = c0 * 8;
    cs = std::min((c1 - c0) * 8, P.K / 32 - s_begin);
    const int p0 = parent * P.steps / S, p1 = (parent + 1) * P.steps / S;
    pb = p0 * 8;
    pcs = std::min((p1 - p0) * 8, P.K / 32 - pb);
}

// The order in which each workgroup of a pass runs units: the host
// simulates the launch with a plain cost model (a unit costs its weight
// bytes at one workgroup's streaming rate; a phase whose input another
// phase writes starts a hand-off after that phase's last unit; staging an
// input chunk costs a fixed time that grows with M) and gives every unit,
// phase by phase, to the workgroup that can start it first, preferring one
// that has its input chunk staged already.  Within a phase the units go out
// last to first, so the finely cut units of a balanced phase run first and
// each workgroup ends the phase on a unit whose tile needs no combine.
// A phase that no phase waits for (no reader) is placed after the phase
// that follows it: each of its units goes into a workgroup's idle gap
// before that workgroup turns to the next phase (the time it would start
// waiting for that phase's input, or the hand-off after that phase for a
// workgroup with no unit in it), and only a unit that fits no gap delays
// a later unit, where it delays least.  Its entries go in front of the next
// phase's, so each workgroup's list stays in phase order and every wait is
// for an earlier phase: the launch cannot deadlock whatever the model gets
// wrong; the model only decides how well the work is spread.
static void schedule(const std::vector<PhaseDesc> &host, const std::vector<int> &producer, int M, int G,
                     std::vector<uint32_t> &out) {
    const int n = static_cast<int>(host.size());
    // per workgroup: streaming rate in bytes per microsecond, and the fixed
    // costs of a unit, a hand-off and a staged chunk in microseconds
    const double rate = 26000.0 / (1.0 + 0.13 * (M - 1));
    const double unit_ovh = 0.5, hand = 1.0, stage = 1.1 + 0.18 * (M - 1);
    std::vector<int> readers(n, 0);
    for (int p = 0; p < n; p++)
        if (producer[p] >= 0) readers[producer[p]]++;
    std::vector<double> free_at(G, 0.0), phase_end(n, 0.0);
    struct Staged {
        const void *in = nullptr;
        int b = -1, c = 0;
    };
    std::vector<Staged> st(G);
    std::vector<std::vector<uint32_t>> lists(G);
    auto ready_of = [&](int p) { return producer[p] >= 0 ? phase_end[producer[p]] + hand : 0.0; };
    struct UnitModel {
        double cost;
        int sb, cs, pb, pcs;
    };
    auto model = [&](const PhaseDesc &P, uint32_t u) {
        UnitModel m;
        int c0, c1;
        host_unit_range(P, u, c0, c1, m.sb, m.cs, m.pb, m.pcs);
        const double row_bytes = static_cast<double>(P.bbytes) / 16.0 * (P.fused ? 2.0 : 1.0);
        m.cost = kRows * (c1 - c0) * row_bytes / rate + unit_ovh;
        return m;
    };
    auto staged = [](const Staged &s, const PhaseDesc &P, const UnitModel &m) {
        return s.in == P.aq && m.sb >= s.b && m.sb + m.cs <= s.b + s.c;
    };
    auto place = [&](int p) {
        const PhaseDesc &P = host[p];
        const double ready = ready_of(p);
        // the units of tiles cut finer than S chunks (the last ones) are
        // given out first: their partial sums are combined while the whole
        // units run, so a phase ends on units that need no combine
        for (int ui = P.n_units - 1; ui >= 0; ui--) {
            const UnitModel m = model(P, static_cast<uint32_t>(ui));
            int best = 0;
            double best_t = 1e300;
            bool best_staged = false;
            for (int w = 0; w < G; w++) {
                const bool sg = staged(st[w], P, m);
                const double t0 = std::max(free_at[w], ready) + (sg ? 0.0 : stage);
                // of equal starts, the workgroup idle longest: so a narrow
                // phase does not land on the workgroups that ran the narrow
                // phase before it, and the idle gaps alternate
                if (t0 < best_t - 1e-9 || (t0 < best_t + 1e-9 && free_at[w] < free_at[best] - 1e-9)) {
                    best_t = t0;
                    best = w;
                    best_staged = sg;
                }
            }
            if (!best_staged) st[best] = {P.aq, m.pb, m.pcs};
            free_at[best] = best_t + m.cost;
            phase_end[p] = std::max(phase_end[p], free_at[best]);
            lists[best].push_back(static_cast<uint32_t>(p) << 20 | static_cast<uint32_t>(ui));
        }
    };
    // the units of phase d (no reader) around phase p = d + 1, already placed
    // from the state `gap`, `gst` (free times and staged chunks before p)
    auto fill = [&](int d, int p, const std::vector<double> &gap, const std::vector<Staged> &gst,
                    const std::vector<size_t> &mark) {
        const PhaseDesc &D = host[d];
        const double ready = ready_of(d), ready_p = ready_of(p);
        std::vector<double> cur(gap), deadline(G);
        std::vector<Staged> cst(gst);
        std::vector<size_t> ins(G, 0);
        std::vector<bool> has_p(G);
        for (int w = 0; w < G; w++) {
            has_p[w] = lists[w].size() > mark[w];
            deadline[w] = has_p[w] ? std::max(gap[w], ready_p) : phase_end[p] + hand;
        }
        for (int ui = D.n_units - 1; ui >= 0; ui--) {
            const UnitModel m = model(D, static_cast<uint32_t>(ui));
            int best = 0;
            double best_over = 1e300, best_t = 1e300;
            bool best_staged = false;
            for (int w = 0; w < G; w++) {
                const bool sg = staged(cst[w], D, m);
                const double t0 = std::max(cur[w], ready) + (sg ? 0.0 : stage);
                const double over = std::max(0.0, t0 + m.cost - deadline[w]);
                if (over < best_over - 1e-9 || (over < best_over + 1e-9 && t0 < best_t - 1e-9)) {
                    best_over = over;
                    best_t = t0;
                    best = w;
                    best_staged = sg;
                }
            }
            if (!best_staged) cst[best] = {D.aq, m.pb, m.pcs};
            cur[best] = best_t + m.cost;
            phase_end[d] = std::max(phase_end[d], cur[best]);
            lists[best].insert(lists[best].begin() + static_cast<std::ptrdiff_t>(mark[best] + ins[best]++),
                               static_cast<uint32_t>(d) << 20 | static_cast<uint32_t>(ui));
        }
        // a workgroup whose gap overflowed runs its later units that much later
        for (int w = 0; w < G; w++) {
            if (!ins[w]) continue;
            if (has_p[w]) {
                const double over = std::max(0.0, cur[w] - deadline[w]);
                free_at[w] += over;
                phase_end[p] = std::max(phase_end[p], free_at[w]);
            } else {
                free_at[w] = std::max(free_at[w], cur[w]);
                st[w] = cst[w];
            }
        }
    };
    for (int p = 0; p < n; p++) {
        if (readers[p] == 0 && p + 1 < n) {
            // phase p waits until phase p + 1 is placed
            std::vector<double> gap(free_at);
            std::vector<Staged> gst(st);
            std::vector<size_t> mark(G);
            for (int w = 0; w < G; w++) mark[w] = lists[w].size();
            place(p + 1);
            fill(p, p + 1, gap, gst, mark);
            p++;
            continue;
        }
        place(p);
    }
    out.assign(static_cast<size_t>(G) + 1, 0u);
    for (int w = 0; w < G; w++) out[w + 1] = out[w] + static_cast<uint32_t>(lists[w].size());
    for (int w = 0; w < G; w++) out.insert(out.end(), lists[w].begin(), lists[w].end());
}

// Every (phase, unit) exactly once, each list in phase order: what the
// kernel relies on for in-range units and for waits that always end.
static bool schedule_ok(const std::vector<PhaseDesc> &host, int G, const std::vector<uint32_t> &s) {
    if (s.size() < static_cast<size_t>(G) + 1) return false;
    size_t total = 0;
    std::vector<size_t> base(host.size() + 1, 0);
    for (size_t p = 0; p < host.size(); p++) base[p + 1] = base[p] + static_cast<size_t>(host[p].n_units);
    total = base.back();
    if (s[G] != total || s.size() != static_cast<size_t>(G) + 1 + total) return false;
    std::vector<uint8_t> seen(total, 0);
    for (int w = 0; w < G; w++) {
        if (s[w] > s[w + 1]) return false;
        int prev = -1;
        for (uint32_t i = s[w]; i < s[w + 1]; i++) {
            const uint32_t e = s[G + 1 + i];
            const int p = static_cast<int>(e >> 20);
            const uint32_t u = e & 0xFFFFFu;
            if (p >= static_cast<int>(host.size()) || p < prev || u >= static_cast<uint32_t>(host[p].n_units))
                return false;
            if (seen[base[p] + u]++) return false;
            prev = p;
        }
    }
    return true;
}

struct Span {
    uintptr_t a, b;   // [a, b) widened to 256-byte blocks
    int phase;
};

static Span span_of(const void *p, size_t bytes, int phase) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p) & ~static_cast<uintptr_t>(255);
    const uintptr_t b = (reinterpret_cast<uintptr_t>(p) + bytes + 255) & ~static_cast<uintptr_t>(255);
    return {a, b, phase};
}

// Dependencies and buffer rules of a pass:
//  * each phase's requantised outputs (q, d, s16, sumsq) have 256-byte
//    blocks of their own: every consumer reads them through its cache
//    level, which can hold no stale copy of a block written once per launch;
//  * a phase's input is either exactly the outputs of an earlier phase (its
//    producer, which it waits for) or shares no block with anything the
//    launch writes.
static int link_phases(std::vector<PhaseDesc> &host, int M, std::vector<int> &producer) {
    const int n = static_cast<int>(host.size());
    producer.assign(n, -1);
    std::vector<Span> outs;
    for (int i = 0; i < n; i++) {
        const PhaseDesc &P = host[i];
        if (P.ep_mode != SV_EP_NONE) {
            const size_t N = static_cast<size_t>(P.N);
            outs.push_back(span_of(P.oq, M * N, i));
            outs.push_back(span_of(P.od, M * N / 8, i));
            outs.push_back(span_of(P.os16, M * N / 4, i));
            outs.push_back(span_of(P.osumsq, M * N / 8, i));
        }
    }
    std::vector<Span> sorted = outs;
    std::sort(sorted.begin(), sorted.end(), [](const Span &x, const Span &y) { return x.a < y.a; });
    for (size_t i = 1; i < sorted.size(); i++)
        SV_REQUIRE(sorted[i].a >= sorted[i - 1].b, SV_ERR_ARG,
                   "pass_create: requantised outputs (phases " + std::to_string(sorted[i - 1].phase) + " and " +
                       std::to_string(sorted[i].phase) + ") share 256-byte blocks; every one needs buffers of its own");
    // everything else the launch writes: y outputs and argmax words
    std::vector<Span> written = outs;
    for (int i = 0; i < n; i++) {
        const PhaseDesc &P = host[i];
        for (int j = 0; j < P.n_w; j++)
            if (P.y[j]) written.push_back(span_of(P.y[j], static_cast<size_t>(M) * P.N * 4, i));
        if (P.argmax) written.push_back(span_of(P.argmax, static_cast<size_t>(M) * 8, i));
    }
    for (int i = 0; i < n; i++) {
        PhaseDesc &P = host[i];
        int prod = -1;
        for (int j = i - 1; j >= 0 && prod < 0; j--)
            if (host[j].ep_mode != SV_EP_NONE && host[j].oq == P.aq) prod = j;
        if (prod >= 0) {
            const PhaseDesc &Q = host[prod];
            SV_REQUIRE(Q.N == P.K && Q.od == P.ad && Q.os16 == P.as16 &&
                           (P.in_parts == nullptr || P.in_parts == Q.osumsq),
                       SV_ERR_ARG,
                       "pass_create: phase " + std::to_string(i) + " reads phase " + std::to_string(prod) +
                           "'s codes but not exactly its scales, sums and partials");
            producer[i] = prod;
            continue;
        }
        const Span ins[4] = {span_of(P.aq, static_cast<size_t>(M) * P.K, i),
                             span_of(P.ad, static_cast<size_t>(M) * P.K / 8, i),
                             span_of(P.as16, static_cast<size_t>(M) * P.K / 4, i),
                             P.in_parts ? span_of(P.in_parts, static_cast<size_t>(M) * P.n_parts * 4, i)
                                        : Span{0, 0, i}};
        for (const Span &s : ins)
            for (const Span &w : written)
                SV_REQUIRE(s.b <= w.a || w.b <= s.a, SV_ERR_ARG,
                           "pass_create: the input of phase " + std::to_string(i) +
                               " shares 256-byte blocks with an output of phase " + std::to_string(w.phase) +
                               " without being that phase's requantised output");
    }
    return SV_OK;
}

}  // namespace sv

extern "C" size_t sv_pass_workspace_bytes(const sv_phase *phases, int32_t n_phases) {
    std::vector<sv::PhaseDesc> host;
    sv::PassLayout L;
    if (sv::plan_pass(phases, n_phases, host, L) != SV_OK) return 0;
    return L.total;
}

extern "C" size_t sv_pass_schedule(const sv_phase *phases, int32_t n_phases, int32_t grid, uint32_t *out,
                                   size_t cap) {
    using namespace sv;
    std::vector<PhaseDesc> host;
    PassLayout L;
    if (plan_pass(phases, n_phases, host, L) != SV_OK) return 0;
    if (grid < 1 || grid > kMaxGrid) {
        fail(SV_ERR_ARG, "pass_schedule: grid must be in [1, " + std::to_string(kMaxGrid) + "]");
        return 0;
    }
    const int M = phases[0].A.M;
    std::vector<int> producer;
    if (link_phases(host, M, producer) != SV_OK) return 0;
    std::vector<uint32_t> plan;
    schedule(host, producer, M, grid, plan);
    if (!schedule_ok(host, grid, plan)) {
        fail(SV_ERR_ARG, "pass_schedule: internal error: inconsistent schedule");
        return 0;
    }
    if (out) {
        if (cap < plan.size()) {
            fail(SV_ERR_ARG, "pass_schedule: out holds " + std::to_string(cap) + " words, the lists need " +
                                 std::to_string(plan.size()));
            return 0;
        }
        std::copy(plan.begin(), plan.end(), out);
    }
    return plan.size();
}

extern "C" int sv_pass_create(const sv_phase *phases, int32_t n_phases, void *workspace, size_t ws_bytes,
                              sv_pass **out) {
    using namespace sv;
    SV_REQUIRE(out, SV_ERR_ARG, "pass_create: out is NULL");
    *out = nullptr;
    std::vector<PhaseDesc> host;
    PassLayout L;
    int rc = plan_pass(phases, n_phases, host, L);
    if (rc) return rc;
    SV_REQUIRE(workspace && ws_bytes >= L.total, SV_ERR_WORKSPACE,
               "pass_create: workspace needs " + std::to_string(L.total) + " bytes");
    SV_REQUIRE(aligned(workspace, 256), SV_ERR_ALIGN, "pass_create: workspace must be 256-byte aligned");
    const int M = phases[0].A.M;
    std::vector<int> producer;
    rc = link_phases(host, M, producer);
    if (rc) return rc;
    uint8_t *b = static_cast<uint8_t *>(workspace);
    uint32_t *sched = reinterpret_cast<uint32_t *>(b + L.table);
    unsigned *ctl = reinterpret_cast<unsigned *>(b + L.table + L.sched);
    uint8_t *scratch = b + L.table + L.sched + L.ctl + L.trace;
    ArgmaxList am{};
    std::vector<int> readers(n_phases, 0);
    for (int i = 0; i < n_phases; i++)
        if (producer[i] >= 0) readers[producer[i]]++;
    for (int i = 0; i < n_phases; i++) {
        PhaseDesc &P = host[i];
        if (needs_partials(P)) {
            P.tile_count = reinterpret_cast<unsigned *>(scratch + L.tiles_off[i]);
            P.partial = reinterpret_cast<float *>(scratch + L.part_off[i]);
        }
        // The readers of a phase read only its requantised output: with K
        // unsplit and no pairing, that comes from the units of matrix
        // ep_src alone.
        P.count_all = (P.S1 > 1 || P.ep_mode != SV_EP_QUANT) ? 1 : 0;
        P.ready = readers[i] ? ctl + kSlotStride * (1 + i * kPhaseCounters) : nullptr;
        if (P.argmax) {
            SV_REQUIRE(am.n < kMaxArgmax, SV_ERR_ARG, "pass_create: at most 4 phases may have an argmax");
            am.p[am.n] = P.argmax;
            am.M[am.n] = M;
            am.n++;
        }
    }
    for (int i = 0; i < n_phases; i++) {
        PhaseDesc &P = host[i];
        P.wait = nullptr;
        P.wait_target = 0u;
        if (producer[i] < 0) continue;
        const PhaseDesc &Q = host[producer[i]];
        P.wait = Q.ready;
        P.wait_target = static_cast<uint32_t>(Q.count_all ? Q.n_units : Q.n_tiles);
    }
    rc = place_parts(host.data(), n_phases, M);
    if (rc) return rc;
    int chunk = 0, np = 0;
    size_t lds = 0;
    for (auto &P : host) {
        chunk = std::max(chunk, P.chunk_sub);
        np = std::max(np, P.n_parts);
        lds = std::max(lds, phase_lds(P, M));
    }
    lds += wpart_bytes(M);
    rc = prepare_lds(M, lds);
    if (rc) return rc;
    int dev = 0;
    hipDeviceProp_t prop;
    rc = hip_check(hipGetDevice(&dev), "pass_create");
    if (!rc) rc = hip_check(hipGetDeviceProperties(&prop, dev), "pass_create");
    if (rc) return rc;
    // Every workgroup of the pass must be resident at once (they wait on each
    // other's phases): the grid is what the GPU holds of this kernel.
    const int occ = resident_per_cu(M, lds, prop, kOccFns[M - 1](lds));
    SV_REQUIRE(occ >= 1, SV_ERR_HIP, "pass_create: the pass kernel cannot be resident with this LDS size");
    sv_pass *p = new sv_pass();
    p->M = M;
    p->n_phases = n_phases;
    p->CS = chunk;
    p->NP = np;
    p->lds = lds;
    p->table = reinterpret_cast<PhaseDesc *>(b);
    p->sched = sched;
    p->ctl = ctl;
    p->trace = reinterpret_cast<unsigned long long *>(b + L.table + L.sched + L.ctl);
    p->tracing = false;
    p->am = am;
    p->host = std::move(host);
    p->grid = std::min(prop.multiProcessorCount * std::min(occ, 2), kMaxGrid);
    std::vector<uint32_t> plan;
    schedule(p->host, producer, M, p->grid, plan);
    if (!schedule_ok(p->host, p->grid, plan)) {
        delete p;
        return fail(SV_ERR_ARG, "pass_create: internal error: inconsistent schedule");
    }
    rc = hip_check(hipMemcpy(p->table, p->host.data(), static_cast<size_t>(n_phases) * sizeof(PhaseDesc),
                             hipMemcpyHostToDevice),
                   "pass_create upload");
    if (!rc)
        rc = hip_check(hipMemcpy(sched, plan.data(), plan.size() * 4, hipMemcpyHostToDevice), "pass_create schedule");
    if (!rc) rc = hip_check(hipMemset(p->ctl, 0, L.ctl), "pass_create ctl");
    if (!rc) rc = hip_check(hipMemset(p->trace, 0, L.trace), "pass_create trace");
    if (!rc && L.scratch) rc = hip_check(hipMemset(scratch, 0, L.scratch), "pass_create scratch");
    if (!rc) rc = hip_check(hipDeviceSynchronize(), "pass_create");
    if (rc) {
        delete p;
        return rc;
    }
    *out = p;
    return SV_OK;
}

extern "C" int sv_pass_run(const sv_pass *p, void *stream) {
    using namespace sv;
    SV_REQUIRE(p, SV_ERR_ARG, "pass_run: NULL pass");
    hipStream_t st = as_stream(stream);
    kPassFns[p->M - 1](p->grid, p->lds, st, p->table, p->n_phases, p->sched, p->ctl, p->CS, p->am,
                       p->tracing ? p->trace : nullptr);
    return hip_check(hipGetLastError(), "pass_run launch");
}

extern "C" int sv_pass_status(const sv_pass *p, uint32_t *status) {
    SV_REQUIRE(p && status, SV_ERR_ARG, "pass_status: NULL argument");
    int rc = sv::hip_check(hipDeviceSynchronize(), "pass_status");
    if (!rc) rc = sv::hip_check(hipMemcpy(status, p->ctl + sv::kCtlResult, 4, hipMemcpyDeviceToHost), "pass_status");
    if (!rc && *status) rc = sv::hip_check(hipMemset(p->ctl + sv::kCtlResult, 0, 4), "pass_status");
    return rc;
}

extern "C" int sv_pass_trace(sv_pass *p, int enable, uint64_t *host, size_t bytes, int32_t *grid) {
    using namespace sv;
    SV_REQUIRE(p, SV_ERR_ARG, "pass_trace: NULL pass");
    p->tracing = enable != 0;
    if (grid) *grid = p->grid;
    if (!host) return SV_OK;
    const size_t need = static_cast<size_t>(p->grid) * p->n_phases * kTraceWords * 8;
    SV_REQUIRE(bytes >= need, SV_ERR_WORKSPACE, "pass_trace: host buffer needs " + std::to_string(need) + " bytes");
    return hip_check(hipMemcpy(host, p->trace, need, hipMemcpyDeviceToHost), "pass_trace");
}

extern "C" void sv_pass_destroy(sv_pass *p) { delete p; }
