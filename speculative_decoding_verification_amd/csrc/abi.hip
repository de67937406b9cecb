// abi.hip - error reporting, version, and stream-layout helpers of the C ABI.
#include <string>

#include "sv_internal.h"

namespace sv {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

int hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return SV_OK;
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return SV_ERR_HIP;
}

// Repacked layout: independent streams, each row-major with one fixed-size
// record per row per block, laid out one after another.  Every stream
// starts at a 16-byte multiple for the shapes the calls accept.
bool streams_of(int32_t qtype, int64_t rows, int64_t cols, Streams *s) {
    if (rows <= 0 || cols <= 0) return false;
    const size_t R = static_cast<size_t>(rows), C = static_cast<size_t>(cols);
    for (int i = 0; i < 4; i++) s->off[i] = 0;
    switch (qtype) {
    case SV_Q8_0:
        if (C % 32) return false;
        s->off[0] = 0;              // int8 quants [R][C]
        s->off[1] = R * C;          // fp16 d [R][C/32]
        s->total = R * C + R * (C / 32) * 2;
        return true;
    case SV_Q4_K:
        if (C % 256) return false;
        s->off[0] = 0;                        // 16-byte quant records [R][C/32]
        s->off[1] = R * (C / 32) * 16;        // 16-byte headers [R][C/256]
        s->total = s->off[1] + R * (C / 256) * 16;
        return true;
    case SV_Q6_K:
        if (C % 256) return false;
        s->off[0] = 0;                        // low nibbles [R][C/32] x 16 B
        s->off[1] = R * (C / 32) * 16;        // high bits  [R][C/32] x 8 B
        s->off[2] = s->off[1] + R * (C / 32) * 8;   // int8 scales [R][C/16]
        s->off[3] = s->off[2] + R * (C / 16);       // fp16 d [R][C/256]
        s->total = s->off[3] + R * (C / 256) * 2;
        return true;
    default:
        return false;
    }
}

}  // namespace sv

extern "C" {

const char *sv_last_error(void) { return sv::g_last_error.c_str(); }

const char *sv_version(void) { return "specverify 0.1 (gfx950)"; }

size_t sv_repacked_bytes(int32_t qtype, int64_t rows, int64_t cols) {
    sv::Streams s;
    if (!sv::streams_of(qtype, rows, cols, &s)) return 0;
    return s.total;
}

int64_t sv_argmax_index(uint64_t packed) {
    return static_cast<int64_t>(0xFFFFFFFFull - (packed & 0xFFFFFFFFull));
}

}  // extern "C"
