// measure.hip - a pure-read kernel: the HBM read rate the box achieves with
// a plain streaming loop, the context the weight-stream rate of a pass is
// reported against.  Not a step of the verification pass.
#include "sv_internal.h"

namespace sv {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;   // 16-byte loads in flight per thread

// Workgroup g reads 16-byte words g*T*U + t + k*T (k < U), then strides by
// the grid; every word is read once.  The XOR of what a workgroup read goes
// to sink[g], so the loads cannot be dropped.
__global__ __launch_bounds__(kReadThreads) void read_kernel(const uint4 *__restrict__ src, int64_t words,
                                                            uint32_t *__restrict__ sink) {
    uint32_t acc = 0;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kReadThreads * kReadUnroll;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kReadThreads * kReadUnroll + threadIdx.x; base < words;
         base += step) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int k = 0; k < kReadUnroll; k++) {
            const int64_t i = base + static_cast<int64_t>(k) * kReadThreads;
            v[k] = i < words ? gld16_nt(src + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kReadUnroll; k++) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o, 64));
    __shared__ uint32_t part[kReadThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace sv

extern "C" int sv_read_bandwidth(const void *src, size_t bytes, uint32_t *sink, int32_t n_sink, void *stream) {
    SV_REQUIRE(src && sink, SV_ERR_ARG, "read_bandwidth: NULL buffer");
    SV_REQUIRE(bytes > 0 && bytes % 16 == 0, SV_ERR_SHAPE, "read_bandwidth: bytes must be a positive multiple of 16");
    SV_REQUIRE(n_sink >= 1 && n_sink <= (1 << 20), SV_ERR_ARG, "read_bandwidth: n_sink must be in [1, 2^20]");
    SV_REQUIRE(sv::aligned(src, 16) && sv::aligned(sink, 4), SV_ERR_ALIGN, "read_bandwidth: alignment");
    hipLaunchKernelGGL(sv::read_kernel, dim3(n_sink), dim3(sv::kReadThreads), 0, sv::as_stream(stream),
                       static_cast<const uint4 *>(src), static_cast<int64_t>(bytes / 16), sink);
    return sv::hip_check(hipGetLastError(), "read_bandwidth launch");
}
