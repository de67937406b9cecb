// sv_internal.h - helpers shared by the HIP sources of libspecverify.
//
// Everything here belongs to the GPU library; nothing is shared with the
// CPU reference used by the tests.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/specverify.h"

namespace sv {

// ----------------------------------------------------------------- errors
void set_error(const std::string &msg);
int fail(int code, const std::string &msg);
int hip_check(hipError_t e, const char *what);

#define SV_REQUIRE(cond, code, msg)                  \
    do {                                             \
        if (!(cond)) return ::sv::fail((code), (msg)); \
    } while (0)

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// ----------------------------------------------------------------- formats
// Repacked stream sizes for a rows x cols matrix (bytes of each stream).
struct Streams {
    size_t off[4];
    size_t total;
};
bool streams_of(int32_t qtype, int64_t rows, int64_t cols, Streams *s);

// --------------------------------------------------------- device helpers
__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    _Float16 h;
    uint16_t b = static_cast<uint16_t>(h16);
    __builtin_memcpy(&h, &b, 2);
    return static_cast<float>(h);
}

__device__ __forceinline__ int32_t dot4(uint32_t a, uint32_t b, int32_t c) {
    return __builtin_amdgcn_sdot4(static_cast<int32_t>(a), static_cast<int32_t>(b), c, false);
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger
// key); -0 is first turned into +0 so the two compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
    f = f + 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long pack_argmax(float f, uint32_t idx) {
    return (static_cast<unsigned long long>(float_key(f)) << 32) |
           static_cast<unsigned long long>(0xFFFFFFFFu - idx);
}

}  // namespace sv
