// repack.hip - load-time rearrangement of GGUF blocks (a1) and its inverse.
//
// The projection kernels read the weights of 16 rows by 256 columns as one
// contiguous block whose fields are stored in the order the lanes read them
// (the layout is described with blocked_of), so every load instruction of a
// wave reads one contiguous range.  GGUF's own blocks (34, 144 and 210
// bytes) are not 16-byte multiples, and Q4_K / Q6_K interleave the nibbles
// of two 32-element sub-blocks in one byte range.  Values never
// change: every field is copied, only moved ("Inside OpenJet Engine: making
// speculative decoding pay", section "One GPU launch for a speculative
// cycle": Q6_K and Q8_0 weights are rearranged at load time for aligned
// access without changing their values; Q4_K gets the same treatment so all
// three formats share one access pattern).
#include "sv_internal.h"

namespace sv {

// 4-bit value of element e (0..255) of a GGUF Q4_K super-block's quants.
__device__ __forceinline__ uint32_t q4k_nib(const uint8_t *qs, int e) {
    int c = e >> 6, hi = (e >> 5) & 1, l = e & 31;
    return (qs[32 * c + l] >> (4 * hi)) & 15u;
}

// Low 4 and high 2 bits of element e of a GGUF Q6_K super-block.
__device__ __forceinline__ uint32_t q6k_lo(const uint8_t *ql, int e) {
    int h = e >> 7, r = e & 127, g = r >> 5, l = r & 31;
    return (ql[64 * h + l + 32 * (g & 1)] >> (g < 2 ? 0 : 4)) & 15u;
}
__device__ __forceinline__ uint32_t q6k_hi(const uint8_t *qh, int e) {
    int h = e >> 7, r = e & 127, g = r >> 5, l = r & 31;
    return (qh[32 * h + l] >> (2 * g)) & 3u;
}

// One thread per (row, step) of the padded matrix: the row's pieces of the
// block (row >> 4, step) are written from the GGUF super-block (or the 8
// Q8_0 blocks) of that row and step; rows past the matrix and Q8_0
// sub-blocks past K are written as zeros.  The inverse reads them back.
__device__ __forceinline__ void blk_pos(int64_t i, int64_t steps, int64_t &row, int64_t &step) {
    row = i / steps;
    step = i - row * steps;
}

__global__ void repack_q8_0(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t rows,
                            int64_t cols, int64_t n, int64_t steps) {
    const int64_t nsub = cols / 32;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t row, st;
        blk_pos(i, steps, row, st);
        uint8_t *blk = dst + ((row >> 4) * steps + st) * 4352;
        const int r = static_cast<int>(row & 15);
        for (int j = 0; j < 8; j++) {
            const int64_t s = st * 8 + j;
            const bool ok = row < rows && s < nsub;
            // rows and blocks past the matrix read block 0 (always valid) and write zeros
            const uint8_t *b = ok ? src + (row * nsub + s) * 34 : src;
            uint8_t *lo = blk + blk_q80_lo(r, j);
            for (int k = 0; k < 16; k++) {
                lo[k] = ok ? b[2 + k] : 0;
                lo[1024 + k] = ok ? b[18 + k] : 0;
            }
            uint8_t *d = blk + blk_q80_d(r, j) + (r & 1) * 2;
            d[0] = ok ? b[0] : 0;
            d[1] = ok ? b[1] : 0;
        }
    }
}

__global__ void unpack_q8_0(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t rows,
                            int64_t cols, int64_t n, int64_t steps) {
    const int64_t nsub = cols / 32;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t row, st;
        blk_pos(i, steps, row, st);
        if (row >= rows) continue;
        const uint8_t *blk = src + ((row >> 4) * steps + st) * 4352;
        const int r = static_cast<int>(row & 15);
        for (int j = 0; j < 8; j++) {
            const int64_t s = st * 8 + j;
            if (s >= nsub) break;
            uint8_t *b = dst + (row * nsub + s) * 34;
            const uint8_t *lo = blk + blk_q80_lo(r, j);
            for (int k = 0; k < 16; k++) {
                b[2 + k] = lo[k];
                b[18 + k] = lo[1024 + k];
            }
            const uint8_t *d = blk + blk_q80_d(r, j) + (r & 1) * 2;
            b[0] = d[0];
            b[1] = d[1];
        }
    }
}

__global__ void repack_q4_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t rows,
                            int64_t n, int64_t steps) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t row, st;
        blk_pos(i, steps, row, st);
        uint8_t *blk = dst + ((row >> 4) * steps + st) * 2304;
        const int r = static_cast<int>(row & 15);
        const bool ok = row < rows;
        const uint8_t *b = ok ? src + (row * steps + st) * 144 : src;
        uint8_t *h = blk + blk_q4k_hdr(r);
        for (int k = 0; k < 16; k++) h[k] = ok ? b[k] : 0;
        const uint8_t *qs = b + 16;
        for (int j = 0; j < 8; j++) {
            uint8_t *rec = blk + blk_q4k_codes(r, j);
            for (int k = 0; k < 16; k++)
                rec[k] = ok ? static_cast<uint8_t>(q4k_nib(qs, 32 * j + k) | (q4k_nib(qs, 32 * j + 16 + k) << 4)) : 0;
        }
    }
}

__global__ void unpack_q4_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t rows,
                            int64_t n, int64_t steps) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t row, st;
        blk_pos(i, steps, row, st);
        if (row >= rows) continue;
        const uint8_t *blk = src + ((row >> 4) * steps + st) * 2304;
        const int r = static_cast<int>(row & 15);
        uint8_t *b = dst + (row * steps + st) * 144;
        const uint8_t *h = blk + blk_q4k_hdr(r);
        for (int k = 0; k < 16; k++) b[k] = h[k];
        auto nib = [&](int e) -> uint32_t {
            const uint8_t *rec = blk + blk_q4k_codes(r, e >> 5);
            const int k = e & 31;
            return (k < 16) ? (rec[k] & 15u) : (rec[k - 16] >> 4);
        };
        for (int c = 0; c < 4; c++)
            for (int l = 0; l < 32; l++)
                b[16 + 32 * c + l] = static_cast<uint8_t>(nib(64 * c + l) | (nib(64 * c + 32 + l) << 4));
    }
}

__global__ void repack_q6_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t rows,
                            int64_t n, int64_t steps) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t row, st;
        blk_pos(i, steps, row, st);
        uint8_t *blk = dst + ((row >> 4) * steps + st) * 3360;
        const int r = static_cast<int>(row & 15);
        const bool ok = row < rows;
        const uint8_t *b = ok ? src + (row * steps + st) * 210 : src;
        const uint8_t *ql = b, *qh = b + 128;
        for (int j = 0; j < 8; j++) {
            uint8_t *L = blk + blk_q6k_ql(r, j);
            for (int k = 0; k < 16; k++)
                L[k] = ok ? static_cast<uint8_t>(q6k_lo(ql, 32 * j + k) | (q6k_lo(ql, 32 * j + 16 + k) << 4)) : 0;
            uint8_t *H = blk + blk_q6k_qh(r, j);
            for (int hh = 0; hh < 2; hh++)
                for (int k = 0; k < 4; k++) {
                    uint32_t v = 0;
                    for (int s = 0; s < 4; s++) v |= q6k_hi(qh, 32 * j + 16 * hh + 4 * s + k) << (2 * s);
                    H[4 * hh + k] = ok ? static_cast<uint8_t>(v) : 0;
                }
            uint8_t *S = blk + blk_q6k_sc(r, j) + (r & 1) * 2;
            S[0] = ok ? b[192 + 2 * j] : 0;
            S[1] = ok ? b[192 + 2 * j + 1] : 0;
        }
        uint8_t *d = blk + blk_q6k_d(r) + (r & 1) * 2;
        d[0] = ok ? b[208] : 0;
        d[1] = ok ? b[209] : 0;
    }
}

__global__ void unpack_q6_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t rows,
                            int64_t n, int64_t steps) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t row, st;
        blk_pos(i, steps, row, st);
        if (row >= rows) continue;
        const uint8_t *blk = src + ((row >> 4) * steps + st) * 3360;
        const int r = static_cast<int>(row & 15);
        uint8_t *b = dst + (row * steps + st) * 210;
        for (int k = 0; k < 192; k++) b[k] = 0;
        for (int e = 0; e < 256; e++) {
            const int j = e >> 5, k = e & 31;
            const uint8_t *L = blk + blk_q6k_ql(r, j);
            const uint32_t lo = (k < 16) ? (L[k] & 15u) : (L[k - 16] >> 4);
            const uint8_t *H = blk + blk_q6k_qh(r, j);
            const int hh = k >> 4, k2 = k & 15, s = k2 >> 2, kk = k2 & 3;
            const uint32_t hi = (H[4 * hh + kk] >> (2 * s)) & 3u;
            const int h = e >> 7, rr = e & 127, g = rr >> 5, l = rr & 31;
            b[64 * h + l + 32 * (g & 1)] |= static_cast<uint8_t>(lo << (g < 2 ? 0 : 4));
            b[128 + 32 * h + l] |= static_cast<uint8_t>(hi << (2 * g));
        }
        for (int j = 0; j < 8; j++) {
            const uint8_t *S = blk + blk_q6k_sc(r, j) + (r & 1) * 2;
            b[192 + 2 * j] = S[0];
            b[192 + 2 * j + 1] = S[1];
        }
        const uint8_t *d = blk + blk_q6k_d(r) + (r & 1) * 2;
        b[208] = d[0];
        b[209] = d[1];
    }
}

__global__ void zero_tail(uint8_t *p, int n) {
    if (static_cast<int>(threadIdx.x) < n) p[threadIdx.x] = 0;
}

static int repack_common(int32_t qtype, const void *src, void *dst, int64_t rows, int64_t cols, void *stream,
                         bool forward) {
    SV_REQUIRE(src && dst, SV_ERR_ARG, "repack: NULL buffer");
    SV_REQUIRE(qtype == SV_Q8_0 || qtype == SV_Q4_K || qtype == SV_Q6_K, SV_ERR_QTYPE,
               "repack: unsupported qtype " + std::to_string(qtype));
    Blocked L;
    SV_REQUIRE(blocked_of(qtype, rows, cols, &L), SV_ERR_SHAPE,
               "repack: cols must be a multiple of 32 (Q8_0) or 256 (Q4_K, Q6_K) and rows > 0");
    SV_REQUIRE(L.total - kTailPad < (static_cast<size_t>(1) << 32), SV_ERR_SHAPE,
               "repack: a repacked matrix must stay under 4 GiB");
    SV_REQUIRE(aligned(forward ? dst : src, 256), SV_ERR_ALIGN, "repack: repacked buffer must be 256-byte aligned");
    const size_t gguf = qtype == SV_Q8_0 ? static_cast<size_t>(rows) * (cols / 32) * 34
                                         : static_cast<size_t>(rows) * (cols / 256) * (qtype == SV_Q4_K ? 144 : 210);
    const uint8_t *a = static_cast<const uint8_t *>(src);
    uint8_t *b = static_cast<uint8_t *>(dst);
    const size_t na = forward ? gguf : L.total, nb = forward ? L.total : gguf;
    SV_REQUIRE(a + na <= b || b + nb <= a, SV_ERR_ARG, "repack: src and dst overlap");
    hipStream_t st = as_stream(stream);
    const int threads = 256;
    const int64_t n = L.hrows * 16 * L.steps;   // (row, step) pairs of the padded matrix
    const int64_t blocks64 = (n + threads - 1) / threads;
    const int blocks = static_cast<int>(blocks64 > 65536 ? 65536 : blocks64);
    if (qtype == SV_Q8_0) {
        if (forward) hipLaunchKernelGGL(repack_q8_0, dim3(blocks), dim3(threads), 0, st, a, b, rows, cols, n, L.steps);
        else hipLaunchKernelGGL(unpack_q8_0, dim3(blocks), dim3(threads), 0, st, a, b, rows, cols, n, L.steps);
    } else if (qtype == SV_Q4_K) {
        if (forward) hipLaunchKernelGGL(repack_q4_k, dim3(blocks), dim3(threads), 0, st, a, b, rows, n, L.steps);
        else hipLaunchKernelGGL(unpack_q4_k, dim3(blocks), dim3(threads), 0, st, a, b, rows, n, L.steps);
    } else {
        if (forward) hipLaunchKernelGGL(repack_q6_k, dim3(blocks), dim3(threads), 0, st, a, b, rows, n, L.steps);
        else hipLaunchKernelGGL(unpack_q6_k, dim3(blocks), dim3(threads), 0, st, a, b, rows, n, L.steps);
    }
    if (forward)
        hipLaunchKernelGGL(zero_tail, dim3(1), dim3(kTailPad), 0, st, b + (L.total - kTailPad),
                           static_cast<int>(kTailPad));
    return hip_check(hipGetLastError(), "repack launch");
}

}  // namespace sv

extern "C" int sv_repack_weights(int32_t qtype, const void *gguf_src, void *dst, int64_t rows, int64_t cols,
                                 void *stream) {
    return sv::repack_common(qtype, gguf_src, dst, rows, cols, stream, true);
}

extern "C" int sv_unpack_weights(int32_t qtype, const void *repacked, void *gguf_dst, int64_t rows,
                                 int64_t cols, void *stream) {
    return sv::repack_common(qtype, repacked, gguf_dst, rows, cols, stream, false);
}
