// repack.hip - load-time rearrangement of GGUF blocks (a1) and its inverse.
//
// The projection kernels read every weight row as fixed-size, aligned
// records (16-byte quant records per 32 elements plus small scale streams),
// so a group of lanes reading consecutive records of one row issues one
// contiguous, 16-byte-aligned load per lane.  GGUF's own blocks (34, 144 and
// 210 bytes) are not 16-byte multiples, and Q4_K / Q6_K interleave the
// nibbles of two 32-element sub-blocks in one byte range.  Values never
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

__global__ void repack_q8_0(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t nblocks,
                            size_t off_d) {
    for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblocks;
         bi += (int64_t)gridDim.x * blockDim.x) {
        const uint8_t *b = src + bi * 34;
        uint8_t *q = dst + bi * 32;
        for (int i = 0; i < 32; i++) q[i] = b[2 + i];
        dst[off_d + bi * 2] = b[0];
        dst[off_d + bi * 2 + 1] = b[1];
    }
}

__global__ void unpack_q8_0(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t nblocks,
                            size_t off_d) {
    for (int64_t bi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; bi < nblocks;
         bi += (int64_t)gridDim.x * blockDim.x) {
        uint8_t *b = dst + bi * 34;
        b[0] = src[off_d + bi * 2];
        b[1] = src[off_d + bi * 2 + 1];
        for (int i = 0; i < 32; i++) b[2 + i] = src[bi * 32 + i];
    }
}

__global__ void repack_q4_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t nsb,
                            size_t off_h) {
    for (int64_t si = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; si < nsb;
         si += (int64_t)gridDim.x * blockDim.x) {
        const uint8_t *b = src + si * 144;
        for (int i = 0; i < 16; i++) dst[off_h + si * 16 + i] = b[i];
        const uint8_t *qs = b + 16;
        for (int j = 0; j < 8; j++) {
            uint8_t *rec = dst + (si * 8 + j) * 16;
            for (int i = 0; i < 16; i++)
                rec[i] = static_cast<uint8_t>(q4k_nib(qs, 32 * j + i) | (q4k_nib(qs, 32 * j + 16 + i) << 4));
        }
    }
}

__global__ void unpack_q4_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t nsb,
                            size_t off_h) {
    for (int64_t si = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; si < nsb;
         si += (int64_t)gridDim.x * blockDim.x) {
        uint8_t *b = dst + si * 144;
        for (int i = 0; i < 16; i++) b[i] = src[off_h + si * 16 + i];
        auto nib = [&](int e) -> uint32_t {
            const uint8_t *rec = src + (si * 8 + (e >> 5)) * 16;
            int i = e & 31;
            return (i < 16) ? (rec[i] & 15u) : (rec[i - 16] >> 4);
        };
        for (int c = 0; c < 4; c++)
            for (int l = 0; l < 32; l++)
                b[16 + 32 * c + l] = static_cast<uint8_t>(nib(64 * c + l) | (nib(64 * c + 32 + l) << 4));
    }
}

__global__ void repack_q6_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t nsb,
                            size_t off_h, size_t off_s, size_t off_d) {
    for (int64_t si = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; si < nsb;
         si += (int64_t)gridDim.x * blockDim.x) {
        const uint8_t *b = src + si * 210;
        const uint8_t *ql = b, *qh = b + 128;
        for (int bb = 0; bb < 8; bb++) {
            uint8_t *L = dst + (si * 8 + bb) * 16;
            for (int i = 0; i < 16; i++)
                L[i] = static_cast<uint8_t>(q6k_lo(ql, 32 * bb + i) | (q6k_lo(ql, 32 * bb + 16 + i) << 4));
            uint8_t *H = dst + off_h + (si * 8 + bb) * 8;
            for (int hh = 0; hh < 2; hh++)
                for (int i = 0; i < 4; i++) {
                    uint32_t v = 0;
                    for (int t = 0; t < 4; t++) v |= q6k_hi(qh, 32 * bb + 16 * hh + 4 * t + i) << (2 * t);
                    H[4 * hh + i] = static_cast<uint8_t>(v);
                }
        }
        for (int k = 0; k < 16; k++) dst[off_s + si * 16 + k] = b[192 + k];
        dst[off_d + si * 2] = b[208];
        dst[off_d + si * 2 + 1] = b[209];
    }
}

__global__ void unpack_q6_k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t nsb,
                            size_t off_h, size_t off_s, size_t off_d) {
    for (int64_t si = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; si < nsb;
         si += (int64_t)gridDim.x * blockDim.x) {
        uint8_t *b = dst + si * 210;
        for (int i = 0; i < 192; i++) b[i] = 0;
        for (int e = 0; e < 256; e++) {
            int bb = e >> 5, i = e & 31;
            const uint8_t *L = src + (si * 8 + bb) * 16;
            uint32_t lo = (i < 16) ? (L[i] & 15u) : (L[i - 16] >> 4);
            const uint8_t *H = src + off_h + (si * 8 + bb) * 8;
            int hh = i >> 4, i2 = i & 15, t = i2 >> 2, ii = i2 & 3;
            uint32_t hi = (H[4 * hh + ii] >> (2 * t)) & 3u;
            int h = e >> 7, r = e & 127, g = r >> 5, l = r & 31;
            b[64 * h + l + 32 * (g & 1)] |= static_cast<uint8_t>(lo << (g < 2 ? 0 : 4));
            b[128 + 32 * h + l] |= static_cast<uint8_t>(hi << (2 * g));
        }
        for (int k = 0; k < 16; k++) b[192 + k] = src[off_s + si * 16 + k];
        b[208] = src[off_d + si * 2];
        b[209] = src[off_d + si * 2 + 1];
    }
}

static int repack_common(int32_t qtype, const void *src, void *dst, int64_t rows, int64_t cols, void *stream,
                         bool forward) {
    SV_REQUIRE(src && dst, SV_ERR_ARG, "repack: NULL buffer");
    SV_REQUIRE(qtype == SV_Q8_0 || qtype == SV_Q4_K || qtype == SV_Q6_K, SV_ERR_QTYPE,
               "repack: unsupported qtype " + std::to_string(qtype));
    Streams s;
    SV_REQUIRE(streams_of(qtype, rows, cols, &s), SV_ERR_SHAPE,
               "repack: cols must be a multiple of 32 (Q8_0) or 256 (Q4_K, Q6_K) and rows > 0");
    SV_REQUIRE(aligned(forward ? dst : src, 256), SV_ERR_ALIGN, "repack: repacked buffer must be 256-byte aligned");
    const uint8_t *a = static_cast<const uint8_t *>(src);
    uint8_t *b = static_cast<uint8_t *>(dst);
    SV_REQUIRE(a + s.total <= b || b + s.total <= a, SV_ERR_ARG, "repack: src and dst overlap");
    hipStream_t st = as_stream(stream);
    const int threads = 256;
    int64_t n = (qtype == SV_Q8_0) ? rows * (cols / 32) : rows * (cols / 256);
    int64_t blocks64 = (n + threads - 1) / threads;
    int blocks = static_cast<int>(blocks64 > 65536 ? 65536 : blocks64);
    if (qtype == SV_Q8_0) {
        if (forward) hipLaunchKernelGGL(repack_q8_0, dim3(blocks), dim3(threads), 0, st, a, b, n, s.off[1]);
        else hipLaunchKernelGGL(unpack_q8_0, dim3(blocks), dim3(threads), 0, st, a, b, n, s.off[1]);
    } else if (qtype == SV_Q4_K) {
        if (forward) hipLaunchKernelGGL(repack_q4_k, dim3(blocks), dim3(threads), 0, st, a, b, n, s.off[1]);
        else hipLaunchKernelGGL(unpack_q4_k, dim3(blocks), dim3(threads), 0, st, a, b, n, s.off[1]);
    } else {
        if (forward)
            hipLaunchKernelGGL(repack_q6_k, dim3(blocks), dim3(threads), 0, st, a, b, n, s.off[1], s.off[2],
                               s.off[3]);
        else
            hipLaunchKernelGGL(unpack_q6_k, dim3(blocks), dim3(threads), 0, st, a, b, n, s.off[1], s.off[2],
                               s.off[3]);
    }
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
