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

bool blocked_of(int32_t qtype, int64_t rows, int64_t cols, Blocked *b) {
    if (rows <= 0 || cols <= 0) return false;
    if (qtype == SV_Q8_0) {
        if (cols % 32) return false;
    } else if (qtype == SV_Q4_K || qtype == SV_Q6_K) {
        if (cols % 256) return false;
    } else {
        return false;
    }
    b->hrows = (rows + 15) / 16;
    b->steps = (cols + 255) / 256;
    b->B = block_bytes(qtype);
    b->total = static_cast<size_t>(b->hrows) * static_cast<size_t>(b->steps) * b->B + kTailPad;
    return true;
}

}  // namespace sv

extern "C" {

const char *sv_last_error(void) { return sv::g_last_error.c_str(); }

const char *sv_version(void) { return "specverify 0.1 (gfx950)"; }

size_t sv_repacked_bytes(int32_t qtype, int64_t rows, int64_t cols) {
    sv::Blocked b;
    if (!sv::blocked_of(qtype, rows, cols, &b)) return 0;
    return b.total;
}

int64_t sv_argmax_index(uint64_t packed) {
    return static_cast<int64_t>(0xFFFFFFFFull - (packed & 0xFFFFFFFFull));
}

}  // extern "C"
