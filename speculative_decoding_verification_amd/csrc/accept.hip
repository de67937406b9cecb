// accept.hip - greedy acceptance (a7) and rejection-sampling acceptance (a8).
//
// Greedy: row i's top token judges draft i; the round keeps the leading
// matches and closes with the top token of the first mismatching row (or
// the last row) ("How Kinetic is fast", section "Why the output does not
// change").
//
// Rejection, all in fp64 ("Speculative Decoding with Open-Weights Models",
// section "Mathematical Integrity: Rejection Sampling for LLMs"; certain
// one-token drafter: "How Kinetic is fast", "Why the output does not
// change"):
//   pass 1  per (row, 1024-chunk): max logit of the chunk (exact);
//   pass 2  per (row, chunk): row max from the chunk maxima, then
//           e_j = exp((z_j - max) / T) and the chunk's sum of e;
//   pass 3  (general drafter) per (row, chunk): S = sum of chunk sums in
//           chunk order, residual r_j = max(0, e_j / S - q_j), chunk sums;
//   pass 4  one workgroup takes the decisions in row order and samples by
//           inverse CDF: the chunk is found from the chunk sums in order,
//           then the index inside it by a prefix scan of recomputed weights.
// Sums are taken in a fixed order, so the result is deterministic; it can
// differ from a strictly sequential fp64 sum only by rounding (~1e-11
// relative for V ~ 1.5e5), i.e. only when a uniform falls that close to a
// decision boundary.
#include <mutex>

#include "sv_internal.h"

namespace sv {

constexpr int kCh = 1024;  // elements per chunk = threads per block

struct AccWs {
    float *cmax;    // [K+1][C]
    double *csum;   // [K+1][C]
    double *rsum;   // [K][C]
};

static size_t ws_layout(int64_t V, int32_t K, size_t *o_cmax, size_t *o_csum, size_t *o_rsum) {
    const size_t C = static_cast<size_t>((V + kCh - 1) / kCh);
    size_t off = 0;
    *o_csum = off;
    off += (K + 1) * C * 8;
    *o_rsum = off;
    off += static_cast<size_t>(K > 0 ? K : 1) * C * 8;
    *o_cmax = off;
    off += (K + 1) * C * 4;
    return (off + 255) / 256 * 256;
}

__device__ float block_max_f32(float v, float *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float r = sh[0];
    for (int w = 1; w < static_cast<int>(blockDim.x >> 6); w++) r = fmaxf(r, sh[w]);
    return r;
}

// Fixed-order block sum: butterfly inside each wave, then wave totals in
// wave order.
__device__ double block_sum_f64(double v, double *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    double r = 0.0;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); w++) r += sh[w];
    return r;
}

__device__ __forceinline__ float row_max(const float *cmax_row, int C) {
    float m = -INFINITY;
    for (int c = 0; c < C; c++) m = fmaxf(m, cmax_row[c]);
    return m;
}

__device__ __forceinline__ double row_total(const double *csum_row, int C) {
    double s = 0.0;
    for (int c = 0; c < C; c++) s += csum_row[c];
    return s;
}

__device__ __forceinline__ double ew(float z, float zmax, double T) {
    return exp((static_cast<double>(z) - static_cast<double>(zmax)) / T);
}

__global__ __launch_bounds__(kCh) void acc_chunk_max(const float *__restrict__ logits, int64_t V, int C,
                                                     float *__restrict__ cmax) {
    __shared__ float sh[16];
    const int c = blockIdx.x, i = blockIdx.y;
    const int64_t j = static_cast<int64_t>(c) * kCh + threadIdx.x;
    const float v = (j < V) ? logits[i * V + j] : -INFINITY;
    const float m = block_max_f32(v, sh);
    if (threadIdx.x == 0) cmax[i * C + c] = m;
}

__global__ __launch_bounds__(kCh) void acc_chunk_sum(const float *__restrict__ logits, int64_t V, int C,
                                                     const float *__restrict__ cmax, double T,
                                                     double *__restrict__ csum) {
    __shared__ double sh[16];
    __shared__ float shm;
    const int c = blockIdx.x, i = blockIdx.y;
    if (threadIdx.x == 0) shm = row_max(cmax + i * C, C);
    __syncthreads();
    const float zmax = shm;
    const int64_t j = static_cast<int64_t>(c) * kCh + threadIdx.x;
    const double e = (j < V) ? ew(logits[i * V + j], zmax, T) : 0.0;
    const double s = block_sum_f64(e, sh);
    if (threadIdx.x == 0) csum[i * C + c] = s;
}

__global__ __launch_bounds__(kCh) void acc_chunk_resid(const float *__restrict__ logits, const float *__restrict__ q,
                                                       int64_t V, int C, const float *__restrict__ cmax,
                                                       const double *__restrict__ csum, double T,
                                                       double *__restrict__ rsum) {
    __shared__ double sh[16];
    __shared__ float shm;
    __shared__ double shS;
    const int c = blockIdx.x, i = blockIdx.y;
    if (threadIdx.x == 0) {
        shm = row_max(cmax + i * C, C);
        shS = row_total(csum + i * C, C);
    }
    __syncthreads();
    const int64_t j = static_cast<int64_t>(c) * kCh + threadIdx.x;
    double r = 0.0;
    if (j < V) {
        const double p = ew(logits[i * V + j], shm, T) / shS;
        const double d = p - static_cast<double>(q[i * V + j]);
        r = d > 0.0 ? d : 0.0;
    }
    const double s = block_sum_f64(r, sh);
    if (threadIdx.x == 0) rsum[i * C + c] = s;
}

struct DecideShared {
    double S[SV_MAX_M];
    float zmax[SV_MAX_M];
    double wsum[16];
    double base;
    int chunk;
    int found;
    int lastnz;
    int accept;
    double thr;
};

// Inverse CDF over the weights of row i: kind 0 = e_j, kind 1 = residual.
// Returns the smallest j whose running sum exceeds thr.
__device__ int64_t sample_row(DecideShared &sh, const float *__restrict__ logits, const float *__restrict__ q,
                              int64_t V, int C, const double *__restrict__ sums, int i, int kind, double thr,
                              double T) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        double acc = 0.0, base_last = 0.0;
        int last = -1, chosen = -1;
        double base = 0.0;
        for (int c = 0; c < C; c++) {
            const double s = sums[i * C + c];
            if (s > 0.0) {
                last = c;
                base_last = acc;
            }
            if (acc + s > thr) {
                chosen = c;
                base = acc;
                break;
            }
            acc += s;
        }
        if (chosen < 0) {
            chosen = last < 0 ? 0 : last;
            base = last < 0 ? 0.0 : base_last;
        }
        sh.chunk = chosen;
        sh.base = base;
        sh.found = 0x7FFFFFFF;
        sh.lastnz = -1;
        sh.thr = thr;
    }
    __syncthreads();
    const int c = sh.chunk;
    const int64_t j = static_cast<int64_t>(c) * kCh + tid;
    double w = 0.0;
    if (j < V) {
        const double e = ew(logits[i * V + j], sh.zmax[i], T);
        if (kind == 0) {
            w = e;
        } else {
            const double d = e / sh.S[i] - static_cast<double>(q[i * V + j]);
            w = d > 0.0 ? d : 0.0;
        }
    }
    // Inclusive scan: within each wave, then wave offsets in wave order.
    const int lane = tid & 63, wave = tid >> 6;
    double v = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) sh.wsum[wave] = v;
    __syncthreads();
    double off = sh.base;
    for (int wv = 0; wv < wave; wv++) off += sh.wsum[wv];
    const double cum = off + v;
    if (j < V && cum > sh.thr) atomicMin(&sh.found, tid);
    if (j < V && w > 0.0) atomicMax(&sh.lastnz, tid);
    __syncthreads();
    int pick = sh.found;
    if (pick == 0x7FFFFFFF) pick = sh.lastnz < 0 ? 0 : sh.lastnz;
    __syncthreads();
    return static_cast<int64_t>(c) * kCh + pick;
}

__global__ __launch_bounds__(kCh) void acc_decide(const float *__restrict__ logits, const float *__restrict__ q,
                                                  int64_t V, int C, const int32_t *__restrict__ drafts, int K,
                                                  const double *__restrict__ u, double T,
                                                  const float *__restrict__ cmax, const double *__restrict__ csum,
                                                  const double *__restrict__ rsum, int32_t *__restrict__ out) {
    __shared__ DecideShared sh;
    const int tid = threadIdx.x;
    if (tid <= K) {
        sh.zmax[tid] = row_max(cmax + tid * C, C);
        sh.S[tid] = row_total(csum + tid * C, C);
    }
    __syncthreads();
    int n = 0;
    for (int i = 0; i <= K; i++) {
        if (q == nullptr) {
            const int64_t t = sample_row(sh, logits, q, V, C, csum, i, 0, u[2 * i] * sh.S[i], T);
            if (i < K && t == drafts[i]) {
                if (tid == 0) out[1 + n] = drafts[i];
                n++;
                continue;
            }
            if (tid == 0) out[1 + n] = static_cast<int32_t>(t);
            break;
        }
        if (i < K) {
            if (tid == 0) {
                const int32_t x = drafts[i];
                int acc = 0;
                if (x >= 0 && x < V) {
                    const double px = ew(logits[i * V + x], sh.zmax[i], T) / sh.S[i];
                    acc = (u[2 * i] * static_cast<double>(q[i * V + x]) < px) ? 1 : 0;
                }
                sh.accept = acc;
            }
            __syncthreads();
            const int accepted = sh.accept;
            __syncthreads();
            if (accepted) {
                if (tid == 0) out[1 + n] = drafts[i];
                n++;
                continue;
            }
            double R = 0.0;
            for (int c = 0; c < C; c++) R += rsum[i * C + c];
            int64_t t;
            if (R > 0.0) t = sample_row(sh, logits, q, V, C, rsum, i, 1, u[2 * i + 1] * R, T);
            else t = sample_row(sh, logits, q, V, C, csum, i, 0, u[2 * i + 1] * sh.S[i], T);
            if (tid == 0) out[1 + n] = static_cast<int32_t>(t);
            break;
        }
        const int64_t t = sample_row(sh, logits, q, V, C, csum, i, 0, u[2 * i + 1] * sh.S[i], T);
        if (tid == 0) out[1 + n] = static_cast<int32_t>(t);
        break;
    }
    if (tid == 0) out[0] = n;
}

// An argmax word of 0 was never written (every packed key has a nonzero
// part), and an index at or beyond n_rows is not a row of the head: either
// makes the round an error (out[0] = -1, every token -1) instead of an index.
__global__ void greedy_kernel(const unsigned long long *__restrict__ argmax, const int32_t *__restrict__ row_ids,
                              int64_t n_rows, const int32_t *__restrict__ drafts, int K, int32_t *__restrict__ out) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int n = 0;
    int32_t tok = 0;
    for (int i = 0; i <= K; i++) {
        const unsigned long long w = argmax[i];
        const int64_t idx = static_cast<int64_t>(0xFFFFFFFFull - (w & 0xFFFFFFFFull));
        if (w == 0ull || idx >= n_rows) {
            for (int j = 0; j < K + 2; j++) out[j] = -1;
            return;
        }
        tok = row_ids ? row_ids[idx] : static_cast<int32_t>(idx);
        if (i < K && drafts[i] == tok) {
            out[1 + n] = tok;
            n++;
            continue;
        }
        break;
    }
    out[1 + n] = tok;
    out[0] = n;
}

}  // namespace sv

extern "C" size_t sv_accept_workspace_bytes(int64_t V, int32_t K) {
    if (V <= 0 || K < 0 || K >= SV_MAX_M) return 0;
    size_t a, b, c;
    return sv::ws_layout(V, K, &a, &b, &c);
}

extern "C" int sv_accept_greedy(const uint64_t *argmax, const int32_t *row_ids, int64_t n_rows, const int32_t *drafts,
                                int32_t K, int32_t *out, void *stream) {
    SV_REQUIRE(argmax && out && (K == 0 || drafts), SV_ERR_ARG, "accept_greedy: NULL buffer");
    SV_REQUIRE(n_rows >= 1 && n_rows < (1ll << 31), SV_ERR_ARG, "accept_greedy: n_rows must be in [1, 2^31)");
    SV_REQUIRE(K >= 0 && K < SV_MAX_M, SV_ERR_ARG, "accept_greedy: K must be in [0, 15]");
    SV_REQUIRE(sv::aligned(argmax, 8) && sv::aligned(out, 4) && (!drafts || sv::aligned(drafts, 4)) &&
                   (!row_ids || sv::aligned(row_ids, 4)),
               SV_ERR_ALIGN, "accept_greedy: alignment");
    hipLaunchKernelGGL(sv::greedy_kernel, dim3(1), dim3(64), 0, sv::as_stream(stream),
                       reinterpret_cast<const unsigned long long *>(argmax), row_ids, n_rows, drafts, K, out);
    return sv::hip_check(hipGetLastError(), "accept_greedy launch");
}

namespace sv {

// The rejection round on a given scratch area (the caller's workspace, or
// the static scratch of the allocation-free entry point).
static int rejection_round(const char *name, const float *logits, int64_t V, const float *q, const int32_t *drafts,
                           int32_t K, const double *u, float temperature, void *workspace, size_t ws_bytes,
                           int32_t *out, void *stream) {
    const std::string who(name);
    SV_REQUIRE(logits && u && out && workspace && (K == 0 || drafts), SV_ERR_ARG, who + ": NULL buffer");
    SV_REQUIRE(K >= 0 && K < SV_MAX_M, SV_ERR_ARG, who + ": K must be in [0, 15]");
    SV_REQUIRE(V >= 1 && V < (1ll << 31), SV_ERR_SHAPE, who + ": V out of range");
    SV_REQUIRE(temperature > 0.0f, SV_ERR_ARG, who + ": temperature must be > 0");
    size_t o_cmax, o_csum, o_rsum;
    const size_t need = ws_layout(V, K, &o_cmax, &o_csum, &o_rsum);
    SV_REQUIRE(ws_bytes >= need, SV_ERR_WORKSPACE, who + ": workspace needs " + std::to_string(need) + " bytes");
    SV_REQUIRE(aligned(workspace, 8) && aligned(logits, 4) && aligned(u, 8) && aligned(out, 4) &&
                   (!q || aligned(q, 4)) && (!drafts || aligned(drafts, 4)),
               SV_ERR_ALIGN, who + ": alignment");
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    float *cmax = reinterpret_cast<float *>(ws + o_cmax);
    double *csum = reinterpret_cast<double *>(ws + o_csum);
    double *rsum = reinterpret_cast<double *>(ws + o_rsum);
    const int C = static_cast<int>((V + kCh - 1) / kCh);
    const double T = static_cast<double>(temperature);
    hipStream_t st = as_stream(stream);
    hipLaunchKernelGGL(acc_chunk_max, dim3(C, K + 1), dim3(kCh), 0, st, logits, V, C, cmax);
    hipLaunchKernelGGL(acc_chunk_sum, dim3(C, K + 1), dim3(kCh), 0, st, logits, V, C, cmax, T, csum);
    if (q && K > 0)
        hipLaunchKernelGGL(acc_chunk_resid, dim3(C, K), dim3(kCh), 0, st, logits, q, V, C, cmax, csum, T, rsum);
    hipLaunchKernelGGL(acc_decide, dim3(1), dim3(kCh), 0, st, logits, q, V, C, drafts, K, u, T, cmax, csum, rsum,
                       out);
    return hip_check(hipGetLastError(), (who + " launch").c_str());
}

// Scratch of the allocation-free entry point: chunk maxima and chunk sums of
// one round, every entry written before it is read within the round, so no
// clearing is needed.  Each GPU holds its own copy until the process ends;
// in host code the array's name only stands in for it, and its device
// address comes from hipGetSymbolAddress with that device current.
constexpr size_t kScratchBytes = 256 * 1024;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch[kMaxDevices];

static int device_scratch(void **out) {
    int dev = 0;
    int rc = hip_check(hipGetDevice(&dev), "accept_rejection_noalloc: device query");
    if (rc) return rc;
    SV_REQUIRE(dev >= 0 && dev < kMaxDevices, SV_ERR_ARG, "accept_rejection_noalloc: device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "accept_rejection_noalloc: scratch address");
        if (rc) return rc;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SV_OK;
}

}  // namespace sv

extern "C" int sv_accept_rejection(const float *logits, int64_t V, const float *q, const int32_t *drafts, int32_t K,
                                   const double *u, float temperature, void *workspace, size_t ws_bytes, int32_t *out,
                                   void *stream) {
    return sv::rejection_round("accept_rejection", logits, V, q, drafts, K, u, temperature, workspace, ws_bytes, out,
                               stream);
}

extern "C" size_t sv_accept_noalloc_max_bytes(void) { return sv::kScratchBytes; }

extern "C" int sv_accept_rejection_noalloc(const float *logits, int64_t V, const float *q, const int32_t *drafts,
                                           int32_t K, const double *u, float temperature, int32_t *out,
                                           void *stream) {
    using namespace sv;
    // sizes first, on the host alone: a round too large for the scratch is
    // refused before any runtime call
    SV_REQUIRE(K >= 0 && K < SV_MAX_M, SV_ERR_ARG, "accept_rejection_noalloc: K must be in [0, 15]");
    SV_REQUIRE(V >= 1 && V < (1ll << 31), SV_ERR_SHAPE, "accept_rejection_noalloc: V out of range");
    size_t a, b, c;
    const size_t need = ws_layout(V, K, &a, &b, &c);
    SV_REQUIRE(need <= kScratchBytes, SV_ERR_WORKSPACE,
               "accept_rejection_noalloc: V = " + std::to_string(V) + ", K = " + std::to_string(K) + " needs " +
                   std::to_string(need) + " bytes of scratch; the static scratch holds " +
                   std::to_string(kScratchBytes) + " (use sv_accept_rejection with a workspace)");
    void *ws = nullptr;
    const int rc = device_scratch(&ws);
    if (rc) return rc;
    return rejection_round("accept_rejection_noalloc", logits, V, q, drafts, K, u, temperature, ws, kScratchBytes,
                           out, stream);
}
