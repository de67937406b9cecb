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
// Repacked weights: one block per (half tile of 16 rows, step of 256
// columns), blocks ordered half tile major, so the rows a wave reads over
// its steps are one contiguous stretch.  Inside a block every field is
// stored lane-major: with lane l = 8 g + j reading rows 2 g, 2 g + 1 of the
// half tile at sub-block j, one load instruction of a field covers one
// contiguous range.  Rows past the matrix (up to a multiple of 16) and
// sub-blocks past K (Q8_0, K not a multiple of 256) are zero, and kTailPad
// zero bytes follow the last block (a load reads up to 8 bytes past a piece).
// Fields per block, for row r (0..15) of the half tile and sub-block j (a
// 2-byte field sits in the dword of its row pair, the even row's in the
// low half, so every small field is read as one aligned dword):
//   Q4_K (2304 B): 16-byte quant records at (r & 1) 1024 + (r >> 1) 128 +
//     16 j, the row's 16-byte super-block header at 2048 + 16 r;
//   Q6_K (3360 B): 16-byte low-nibble records at (r & 1) 1024 + (r >> 1) 128
//     + 16 j, 8-byte high-bit records at 2048 + (r & 1) 512 + (r >> 1) 64 +
//     8 j, the two int8 sub-scales in the dword at 3072 + (r >> 1) 32 + 4 j,
//     fp16 d in the dword at 3328 + (r >> 1) 4;
//   Q8_0 (4352 B): quant bytes 0-15 at (r & 1) 2048 + (r >> 1) 128 + 16 j,
//     bytes 16-31 1024 further, fp16 d in the dword at 4096 + (r >> 1) 32 +
//     4 j.
constexpr size_t kTailPad = 64;
struct Blocked {
    int64_t hrows;    // half tiles (rows rounded up to 16, / 16)
    int64_t steps;    // 256-column steps (cols rounded up to 256, / 256)
    uint32_t B;       // bytes per block
    size_t total;     // hrows * steps * B + kTailPad
};
bool blocked_of(int32_t qtype, int64_t rows, int64_t cols, Blocked *b);

__host__ __device__ inline uint32_t blk_q4k_codes(int r, int j) { return (r & 1) * 1024u + (r >> 1) * 128u + j * 16u; }
__host__ __device__ inline uint32_t blk_q4k_hdr(int r) { return 2048u + r * 16u; }
__host__ __device__ inline uint32_t blk_q6k_ql(int r, int j) { return (r & 1) * 1024u + (r >> 1) * 128u + j * 16u; }
__host__ __device__ inline uint32_t blk_q6k_qh(int r, int j) { return 2048u + (r & 1) * 512u + (r >> 1) * 64u + j * 8u; }
// dword offsets of the 2-byte fields; the row's half is (r & 1)
__host__ __device__ inline uint32_t blk_q6k_sc(int r, int j) { return 3072u + (r >> 1) * 32u + j * 4u; }
__host__ __device__ inline uint32_t blk_q6k_d(int r) { return 3328u + (r >> 1) * 4u; }
__host__ __device__ inline uint32_t blk_q80_lo(int r, int j) { return (r & 1) * 2048u + (r >> 1) * 128u + j * 16u; }
__host__ __device__ inline uint32_t blk_q80_d(int r, int j) { return 4096u + (r >> 1) * 32u + j * 4u; }
__host__ __device__ inline uint32_t block_bytes(int32_t qtype) {
    return qtype == SV_Q4_K ? 2304u : (qtype == SV_Q6_K ? 3360u : 4352u);
}

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
