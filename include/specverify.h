/*
 * specverify.h - C ABI of the speculative-decoding verification pass on
 * AMD Instinct MI355X (gfx950).
 *
 * One call of the pass scores the current token plus K drafted positions of
 * one sequence (M = K + 1 rows, 1 <= M <= 16) in a single stream over
 * GGUF-quantised weights, with int8 activations and integer dot products
 * ("Inside OpenJet Engine: making speculative decoding pay", sections "The
 * bottleneck: reading weights for a small amount of work" and "One GPU
 * launch for a speculative cycle"; "How Kinetic is fast", section "RAD-1:
 * exact speculative decoding").  It ends in a full-vocabulary head whose
 * logits feed greedy or rejection-sampling acceptance.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless a comment says host.  The caller
 *    owns every buffer and passes any scratch space as a workspace; no call
 *    allocates device memory (sv_pass_create allocates one small host
 *    handle).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are asynchronous on it and return only validation / launch
 *    status.  Outputs are ready when the stream has reached the call.
 *  - Arguments are validated before anything is launched; on a non-zero
 *    status nothing was enqueued and sv_last_error() holds a message.
 *  - Layouts are row-major; "[M][K]" means M rows of K contiguous values.
 *  - Results are deterministic, and every output row depends only on its
 *    own input row: a row of an M-row call is bit-identical to the same row
 *    run alone (batch invariance, "How Kinetic is fast", section "Why the
 *    output does not change").
 *  - The library is stateless and thread-safe.  Calls on different streams
 *    may run concurrently if their output buffers do not overlap.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (return value of every int-returning call). */
#define SV_OK 0
#define SV_ERR_ARG (-1)       /* NULL where not allowed, bad mode, M out of range */
#define SV_ERR_SHAPE (-2)     /* a dimension is not a multiple of the block size */
#define SV_ERR_ALIGN (-3)     /* a pointer is not aligned as documented */
#define SV_ERR_QTYPE (-4)     /* unsupported quantisation type */
#define SV_ERR_WORKSPACE (-5) /* workspace too small */
#define SV_ERR_HIP (-6)       /* the HIP runtime reported an error */

/* GGUF tensor type ids of the supported weight formats (the formats ggml
 * defines, "How Kinetic is fast", section "References"). */
#define SV_Q8_0 8  /* 32-element blocks: fp16 d, 32 x int8;          8.5 bits/weight */
#define SV_Q4_K 12 /* 256-element super-blocks: fp16 d, dmin, 6-bit sub-scales and
                      mins per 32, 4-bit quants;                    4.5 bits/weight */
#define SV_Q6_K 14 /* 256-element super-blocks: 6-bit quants, int8 scale per 16,
                      fp16 d;                                       6.5625 bits/weight */

#define SV_MAX_M 16

/* Human-readable text of the last non-OK status on the calling thread. */
const char *sv_last_error(void);

/* Library version string (host memory, static). */
const char *sv_version(void);

/* ------------------------------------------------------------------ */
/* a1. Load-time weight repack.                                        */
/* ------------------------------------------------------------------ */
/* Bytes of the repacked form of a rows x cols matrix of type qtype, or 0
 * for an unsupported type or shape (cols must be a multiple of 32 for Q8_0
 * and of 256 for Q4_K / Q6_K).  The repacked form holds exactly the bytes of
 * the GGUF form (same size), rearranged. */
size_t sv_repacked_bytes(int32_t qtype, int64_t rows, int64_t cols);

/* Rearranges canonical GGUF blocks into the aligned stream layout the
 * projection kernels read, changing no value ("Inside OpenJet Engine",
 * section "One GPU launch for a speculative cycle": Q6_K and Q8_0 weights are
 * rearranged at load time for aligned access without changing their values).
 *   gguf_src: rows x (cols / block) GGUF blocks, contiguous, any alignment.
 *   dst:      sv_repacked_bytes(...) bytes, 256-byte aligned.
 * Layout of dst (all streams row-major, one record per row per block):
 *   Q8_0: int8 quants [rows][cols] | fp16 d [rows][cols/32]
 *   Q4_K: 16-byte quant records [rows][cols/32] (byte i holds elements i and
 *         i+16 of the 32-element sub-block in its low and high nibble) |
 *         the 16-byte super-block headers (d, dmin, packed scales) verbatim
 *         [rows][cols/256]
 *   Q6_K: 16-byte low-nibble records [rows][cols/32] (as Q4_K) | 8-byte
 *         high-bit records [rows][cols/32] (dword h, byte i, bits 2t..2t+1 =
 *         high bits of element 16h + 4t + i) | int8 scales [rows][cols/16] |
 *         fp16 d [rows][cols/256]
 * src and dst must not overlap. */
int sv_repack_weights(int32_t qtype, const void *gguf_src, void *dst, int64_t rows, int64_t cols,
                      void *stream);

/* Inverse of sv_repack_weights (for verification of the load path). */
int sv_unpack_weights(int32_t qtype, const void *repacked, void *gguf_dst, int64_t rows,
                      int64_t cols, void *stream);

/* ------------------------------------------------------------------ */
/* a2. Activation quantiser Q8A32.                                     */
/* ------------------------------------------------------------------ */
/* Per row m and 32-element block b of v = x (times gamma when given, one
 * fp32 rounding per element): amax = max |v|, d = amax / 127 (fp32),
 * id = d ? 1/d : 0, q = clamp(roundf(v * id), -127, 127) (round half away
 * from zero), and the exact int sums of q over each 16-element half
 * ("Inside OpenJet Engine", "One GPU launch...": int8 activations).
 *   x [M][K] fp32, gamma [K] fp32 or NULL, K % 32 == 0, 1 <= M <= 16.
 *   q [M][K] int8, d [M][K/32] fp32, s16 [M][K/16] int32.
 *   sumsq [M][K/32] fp32 or NULL: sum of x^2 (before gamma) of each block,
 *   the partials an RMS norm of x is formed from (see sv_act). */
int sv_quantize_act_q8(const float *x, int32_t M, int64_t K, const float *gamma, int8_t *q,
                       float *d, int32_t *s16, float *sumsq, void *stream);

/* ------------------------------------------------------------------ */
/* a3/a4. Projection of M positions in one weight stream.              */
/* ------------------------------------------------------------------ */
typedef struct {
    int32_t qtype;    /* SV_Q8_0 / SV_Q4_K / SV_Q6_K */
    int64_t rows;     /* output features N */
    int64_t cols;     /* input features K */
    const void *data; /* repacked weights (sv_repack_weights), 256-byte aligned */
} sv_weight;

/* An int8 activation as written by sv_quantize_act_q8 or by an epilogue.
 * When sumsq_parts is given, the input is the RMS-normalised vector
 * r * v with r[m] = 1 / sqrt(sum_i sumsq_parts[m][i] / K + eps); r is
 * folded into every output of the consumer (y = r * W.v_q), so the int8
 * codes never depend on it. */
typedef struct {
    int32_t M;                /* positions, 1..16 */
    int64_t K;                /* features, a multiple of 32, at most 24576 */
    const int8_t *q;          /* [M][K] */
    const float *d;           /* [M][K/32] */
    const int32_t *s16;       /* [M][K/16] */
    const float *sumsq_parts; /* [M][n_parts] or NULL (then r = 1) */
    int32_t n_parts;          /* 1..576 when sumsq_parts is given */
    float eps;
} sv_act;

#define SV_EP_NONE 0  /* write y only */
#define SV_EP_QUANT 1 /* also requantise y[src] * gamma for the next consumer */
#define SV_EP_PAIR 2  /* also requantise (y[0] * y[1]) * gamma (gate x up) */

/* Fused producer epilogue ("Inside OpenJet Engine", "One GPU launch...": the
 * producing phase requantises activations for the next consumer, including
 * the next RMS normalisation's weight).  Output rows must be a multiple of 32.
 * The new activation has K' = rows; its sumsq partials are the per-block sums
 * of the (unnormalised) vector that was quantised, [M][rows/32]. */
typedef struct {
    int32_t mode;       /* SV_EP_* */
    int32_t src;        /* SV_EP_QUANT: which output is requantised */
    const float *gamma; /* [rows] or NULL (= all ones) */
    int8_t *q;          /* [M][rows] */
    float *d;           /* [M][rows/32] */
    int32_t *s16;       /* [M][rows/16] */
    float *sumsq;       /* [M][rows/32] */
} sv_epilogue;

/* Y_j[m][n] = r[m] * sum over 32-blocks b of the exact int32 block sum of
 * weight quants times activation quants, scaled by the block's weight and
 * activation scales (fp32), for each of n_w matrices W[0..n_w-1] that share
 * the input A (q, k, v, or gate, up).  All W[j] have the same qtype and rows,
 * and cols = A->K (matrices of different formats on one input are separate
 * calls, or separate phases of a pass).  y[j] is [M][rows] fp32 or NULL.  ep may be NULL.
 * The K axis is cut into chunks whose number depends only on K and the row
 * count (the tiles of a last partial round of 256 tile-chunks are cut
 * finer); the fp32 combine order (sequential per lane, a fixed tree over a
 * lane group, the step quarters and then the chunks added in order) depends
 * only on K and the row count, never on M, which makes every row
 * batch-invariant and every run deterministic.
 * workspace: sv_matvec_workspace_bytes(W, n_w, A) bytes, 256-byte aligned.
 * Its first 256 KiB hold tile counters that must be zero before the first
 * use; every call leaves them zero again (the rest holds partial sums and
 * needs no initialisation), so one workspace of the largest size can serve
 * calls of any shape.  May be NULL when the size is 0.  Calls sharing a
 * workspace must not run concurrently. */
size_t sv_matvec_workspace_bytes(const sv_weight *W, int32_t n_w, const sv_act *A);
int sv_verify_matvec(const sv_weight *W, int32_t n_w, const sv_act *A, float *const *y,
                     const sv_epilogue *ep, void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* a6/a9. Output head with fused argmax.                               */
/* ------------------------------------------------------------------ */
/* logits[m][i] = projection of row row_ids[i] of H (all rows when row_ids is
 * NULL, then n_rows = H->rows) for input A; the same arithmetic as
 * sv_verify_matvec, so a row's logit does not depend on which other rows are
 * scored ("Inside OpenJet Engine", "Cheap drafting, careful state
 * management": a restricted draft head over a token subset plus tokens added
 * dynamically, while verification keeps the full vocabulary).
 *   row_ids: NULL or n_rows int32 ids in [0, H->rows) (an id outside that
 *   range is a caller error; it is scored as row 0 and never read out of
 *   bounds).
 *   logits [M][n_rows] fp32 or NULL; argmax [M] uint64 or NULL:
 *   argmax[m] = (orderable bits of the max logit) << 32 | (0xFFFFFFFF - i)
 *   for the winning index i (ties go to the lowest i); the token is
 *   row_ids[i] (or i).  sv_argmax_index decodes it on the host.
 *   workspace as for sv_verify_matvec, sv_head_workspace_bytes(H, A, n_rows)
 *   bytes (n_rows = 0 for all rows). */
size_t sv_head_workspace_bytes(const sv_weight *H, const sv_act *A, int64_t n_rows);
int sv_head_logits(const sv_weight *H, const sv_act *A, const int32_t *row_ids, int64_t n_rows,
                   float *logits, uint64_t *argmax, void *workspace, size_t ws_bytes, void *stream);

/* Host helper: index encoded in a packed argmax word. */
int64_t sv_argmax_index(uint64_t packed);

/* ------------------------------------------------------------------ */
/* a5. A whole pass in one persistent launch.                          */
/* ------------------------------------------------------------------ */
/* One phase of a pass: the arguments of one sv_verify_matvec or
 * sv_head_logits call ("Inside OpenJet Engine", "One GPU launch for a
 * speculative cycle": all phases of a cycle in one launch, synchronised
 * between phases, without host round trips).
 * Dependencies follow the buffers: a phase whose A.q is the ep.q of an
 * earlier phase waits for the latest such phase (its producer), and A.d,
 * A.s16 and A.sumsq_parts (if given) must then be that phase's ep.d, ep.s16
 * and ep.sumsq; a phase whose input no earlier phase writes starts at once.
 * So phases that read one input run side by side: on a 27B-class layer,
 * v (Q6_K, requantised for o) and q, k (Q4_K, read by nothing) are two
 * phases on the same input, and o waits for v alone. */
typedef struct {
    const sv_weight *W;      /* n_w matrices (read during sv_pass_create only) */
    int32_t n_w;
    sv_act A;
    float *y[3];
    sv_epilogue ep;          /* ep.mode = SV_EP_NONE for none */
    const int32_t *row_ids;  /* head gather, or NULL */
    int64_t n_rows;
    uint64_t *argmax;        /* head argmax [M], or NULL (at most 4 phases of a pass) */
} sv_phase;

typedef struct sv_pass sv_pass; /* opaque host handle */

/* Device workspace for a pass: phase table, control words, completion
 * counters, trace area, and the tile counters and partial sums of every
 * phase whose tiles are split over units (each phase has its own).  0 if a
 * phase is invalid (sv_last_error() says why). */
size_t sv_pass_workspace_bytes(const sv_phase *phases, int32_t n_phases);

/* Host only, no device call: the unit lists a pass over these phases runs
 * with `grid` workgroups (1..1024), built as sv_pass_create builds them
 * (the same validation, phase links and schedule), for inspecting how the
 * phases of a cycle ("Inside OpenJet Engine: making speculative decoding
 * pay", section "One GPU launch for a speculative cycle") are spread over
 * the workgroups.  The buffers of `phases` are only compared as addresses,
 * never read.  out (host, may be NULL) receives grid + 1 list offsets, then
 * the entries, each (phase << 20) | unit, workgroup w's list being entries
 * [offset[w], offset[w + 1]) in the order it runs them.  Returns the number
 * of 32-bit words (grid + 1 + total units), or 0 with sv_last_error() set
 * if a phase is invalid, grid is out of range or cap is below that number. */
size_t sv_pass_schedule(const sv_phase *phases, int32_t n_phases, int32_t grid, uint32_t *out, size_t cap);

/* Validates every phase (same M for all; buffers as below), writes the
 * phase table into `workspace` (device, 256-byte aligned,
 * sv_pass_workspace_bytes bytes; it must stay allocated and untouched while
 * the pass exists) and returns a small host handle.  Buffer rules, checked
 * here (SV_ERR_ARG otherwise): the requantised outputs (ep.q, d, s16, sumsq)
 * of every phase lie in 256-byte blocks of their own, and a phase's input is
 * either exactly an earlier phase's requantised output or shares no 256-byte
 * block with anything the pass writes (requantised outputs, y, argmax), so
 * no consumer can read a stale cached copy or race a writer.  When several
 * phases write the same y buffer, the pass does not order those writes.
 * This call synchronises with the device; it is load-time work, not per
 * cycle. */
int sv_pass_create(const sv_phase *phases, int32_t n_phases, void *workspace, size_t ws_bytes,
                   sv_pass **out);

/* Enqueues one pass on `stream`: a single persistent launch of as many
 * workgroups as the GPU holds at once (one or two per compute unit, as the
 * launch's registers and LDS allow; one at every M today), each working
 * through its host-built list of units in phase order, that leaves its
 * counters reset for the
 * next run.  Allocates nothing and records no memset, so it can be captured
 * in a graph.  Runs of one pass must not overlap, and the pass expects the
 * GPU to itself while it runs (its workgroups wait on each other; if
 * another kernel keeps some of them from being resident, the waits expire
 * and the run ends early with a nonzero status instead of hanging).  Every
 * argmax of the pass is cleared inside the launch before any head tile adds
 * to it. */
int sv_pass_run(const sv_pass *pass, void *stream);

/* Host: the OR of the status of every run of this pass completed since the
 * previous call (or since sv_pass_create); synchronises the device, then
 * clears it.  0 = every run ok; bit 0 = a wait for a producer phase
 * expired, bit 1 = the wait for the argmax clear expired.  A run that fails
 * has incomplete outputs; the next run still starts clean (the live status
 * word, counters and split tiles are reset at the end of every run). */
int sv_pass_status(const sv_pass *pass, uint32_t *status);

/* Profiling.  enable != 0 makes later runs record, per workgroup and phase,
 * sixteen 64-bit words, [grid][n_phases][16], zero rows for phases in which
 * a workgroup had no unit.  Times are the 100 MHz real-time counter:
 *   0 the workgroup reached the phase;  1 its input was ready;  2 the input
 *   was staged;  3 the first unit's dot products were done (its partial sums
 *   handed to the control wave);  4 the first unit was done (outputs written
 *   and counted);  5 the last unit was done;  6 the number of units it ran;
 *   7 the first unit's rows were combined;  8 its outputs or partial sums
 *   were written;  9 the workgroup's placement (the HW_ID register in the
 *   low 32 bits, XCC_ID in the high 32);  10 the first unit's partial sums
 *   had landed (a tile split over K; else 0);  11 its outputs had landed,
 *   before the hand-off count (0 if no later phase reads it);  12 the
 *   staging transfers were issued;  13 they had landed;  14, 15 unused.
 * Words 1, 2, 12 and 13 describe the workgroup's last staging in the
 * phase (most phases stage once per workgroup).  With host != NULL the last
 * run's record is copied there (synchronous; bytes >= grid * n_phases *
 * 128).  *grid (may be NULL) receives the number of workgroups a run
 * launches. */
int sv_pass_trace(sv_pass *pass, int enable, uint64_t *host, size_t bytes, int32_t *grid);

void sv_pass_destroy(sv_pass *pass);

/* ------------------------------------------------------------------ */
/* a7. Greedy acceptance.                                              */
/* ------------------------------------------------------------------ */
/* Row i's top token judges draft i: n = number of leading drafts equal to
 * the top token of their row; the round emits drafts[0..n-1] and then the
 * top token of row n ("How Kinetic is fast", "Why the output does not
 * change": greedy keeps a guess only when it is the model's top token).
 *   argmax [K+1] packed words from sv_head_logits (or a pass); row_ids and
 *   n_rows as given to it (row_ids NULL: n_rows = the head's rows, and the
 *   index is the token); drafts [K] int32, 0 <= K <= 15.
 *   out [K+2] int32: out[0] = n, out[1..n+1] = emitted tokens.  If a word
 *   that is read was never written (0) or names an index >= n_rows, the
 *   round is an error: out[0] = -1 and every other entry is -1. */
int sv_accept_greedy(const uint64_t *argmax, const int32_t *row_ids, int64_t n_rows,
                     const int32_t *drafts, int32_t K, int32_t *out, void *stream);

/* ------------------------------------------------------------------ */
/* a8. Rejection-sampling acceptance (fp64).                           */
/* ------------------------------------------------------------------ */
/* p_i = softmax(logits_i / temperature) in fp64.
 * General drafter (q != NULL, [K][V] fp32 draft distributions): accept x_i
 * iff u[i][0] * q_i(x_i) < p_i(x_i) (u < min(1, p/q)); on the first rejection
 * emit the smallest j with cumsum_j(max(0, p_i - q_i)) > u[i][1] * R_i (R_i =
 * the residual's total; p_i itself if R_i == 0) and stop; if all K are
 * accepted emit one token from p_K with u[K][1] ("Speculative Decoding with
 * Open-Weights Models", section "Mathematical Integrity: Rejection Sampling
 * for LLMs", the alpha and p' equations).
 * Certain one-token drafter (q == NULL): for i = 0..K, t_i = smallest j with
 * cumsum_j(p_i) > u[i][0]; accept while i < K and t_i == x_i, else emit t_i
 * and stop; this uses one uniform per emitted token in order, so the tokens
 * equal plain sampling with the same uniforms ("How Kinetic is fast", "Why
 * the output does not change").
 *   logits [K+1][V] fp32, drafts [K] int32 (0 <= K <= 15), u [K+1][2] fp64
 *   in [0, 1), temperature > 0, workspace of sv_accept_workspace_bytes(V, K)
 *   bytes (8-byte aligned), out [K+2] int32 as for sv_accept_greedy. */
size_t sv_accept_workspace_bytes(int64_t V, int32_t K);
int sv_accept_rejection(const float *logits, int64_t V, const float *q, const int32_t *drafts,
                        int32_t K, const double *u, float temperature, void *workspace,
                        size_t ws_bytes, int32_t *out, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sv_accept_rejection with
 * the same arguments minus the workspace, run on a static scratch array of
 * sv_accept_noalloc_max_bytes() bytes (256 KiB) that each GPU the library
 * runs on holds until the process ends.  The round must fit it:
 * sv_accept_workspace_bytes(V, K) <= that size (V up to 860160 tokens at
 * K = 15, more for smaller K), else SV_ERR_WORKSPACE before any runtime
 * call.  It allocates nothing; the first call on a device looks up the
 * scratch's address there.  Every call on one GPU shares its scratch, so
 * calls that overlap on one GPU (on different streams, or from several
 * threads without ordering) race and must not be made; the scratch keeps
 * the last call's contents, and a round writes every entry it reads.
 * Results equal sv_accept_rejection's bit for bit. */
size_t sv_accept_noalloc_max_bytes(void);
int sv_accept_rejection_noalloc(const float *logits, int64_t V, const float *q, const int32_t *drafts,
                                int32_t K, const double *u, float temperature, int32_t *out,
                                void *stream);

/* ------------------------------------------------------------------ */
/* Measurement aid (not a step of the pass).                           */
/* ------------------------------------------------------------------ */
/* Reads `bytes` (a multiple of 16) at src once with 16-byte streaming loads
 * in n_sink workgroups and writes the XOR of what workgroup g read to
 * sink[g]: the plain read rate of the device, against which the weight
 * stream of a pass is put in context (src 16-byte aligned, device). */
int sv_read_bandwidth(const void *src, size_t bytes, uint32_t *sink, int32_t n_sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
