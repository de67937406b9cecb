// sv_internal.h - helpers shared by the HIP sources of libspecverify.
//
// Everything here belongs to the GPU library; nothing is shared with the
// CPU reference used by the tests.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "specverify.h"

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
// Global-memory accesses through address-space-1 pointers.  A pointer read
// from memory (a descriptor in LDS, say) is otherwise a generic pointer and
// its loads become flat instructions, which also count against the LDS wait
// counter.  Vector values move as clang vectors, not HIP's vector classes,
// whose copy constructors would take the address back to generic.
#define SV_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T gld(const T *p) {
    return *(const SV_GLOBAL T *)p;
}
template <typename T>
__device__ __forceinline__ void gst(T *p, T v) {
    *(SV_GLOBAL T *)p = v;
}
__device__ __forceinline__ uint4 gld16(const void *p) {
    const u32x4 v = *(const SV_GLOBAL u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 gld8(const void *p) {
    const u32x2 v = *(const SV_GLOBAL u32x2 *)p;
    return make_uint2(v.x, v.y);
}
// Streaming (non-temporal) loads for data read once.
__device__ __forceinline__ uint4 gld16_nt(const void *p) {
    const u32x4 v = __builtin_nontemporal_load((const SV_GLOBAL u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 gld8_nt(const void *p) {
    const u32x2 v = __builtin_nontemporal_load((const SV_GLOBAL u32x2 *)p);
    return make_uint2(v.x, v.y);
}

// Cross-workgroup data of one launch moves through device-coherent accesses
// (written through to, and read from, the level all XCDs share) instead of
// fences: an agent-scope fence writes back or invalidates a whole L2, far too
// costly once per unit.
template <typename T>
__device__ __forceinline__ void st_dev(T *p, T v) {
    __hip_atomic_store((SV_GLOBAL T *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T *p) {
    return __hip_atomic_load((SV_GLOBAL T *)const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T add_dev(T *p, T v) {
    return __hip_atomic_fetch_add((SV_GLOBAL T *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T max_dev(T *p, T v) {
    return __hip_atomic_fetch_max((SV_GLOBAL T *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T or_dev(T *p, T v) {
    return __hip_atomic_fetch_or((SV_GLOBAL T *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's memory operations have completed.
__device__ __forceinline__ void drain() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    _Float16 h;
    uint16_t b = static_cast<uint16_t>(h16);
    __builtin_memcpy(&h, &b, 2);
    return static_cast<float>(h);
}

__device__ __forceinline__ int32_t dot4(uint32_t a, uint32_t b, int32_t c) {
    return __builtin_amdgcn_sdot4(static_cast<int32_t>(a), static_cast<int32_t>(b), c, false);
}
// First product of a dot-product chain, started at c (or at 0): the
// three-operand encoding takes the start value as an operand, where the
// tied two-operand form the compiler picks for the builtin first copies it
// into the accumulator register.
__device__ __forceinline__ int32_t dot4_from(uint32_t a, uint32_t b, int32_t c) {
    int32_t r;
    asm("v_dot4_i32_i8 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ int32_t dot4_first(uint32_t a, uint32_t b) {
    int32_t r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
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
