// quant.hip - activation quantiser Q8A32 (a2).
//
// One 32-lane half-wave quantises one 32-element block: block maximum by a
// butterfly over the half-wave, d = amax / 127 and 1 / d as IEEE fp32
// divisions, codes by round-half-away-from-zero, and the two per-16 code
// sums by integer butterflies (exact, so their order is irrelevant).  The
// per-block sum of x^2 (fp32, fixed butterfly order) feeds the consumer's
// RMS factor ("Inside OpenJet Engine: making speculative decoding pay",
// section "One GPU launch for a speculative cycle": int8 activations).
#include "sv_internal.h"

namespace sv {

__global__ __launch_bounds__(256) void quant_act_kernel(const float *__restrict__ x, const float *__restrict__ gamma,
                                                        int32_t M, int64_t K, int8_t *__restrict__ q,
                                                        float *__restrict__ d, int32_t *__restrict__ s16,
                                                        float *__restrict__ sumsq) {
    const int64_t nb = K / 32;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    if (item >= static_cast<int64_t>(M) * nb) return;  // whole half-wave leaves together
    const int64_t m = item / nb, b = item % nb;
    const float xv = x[m * K + 32 * b + lane];
    const float v = gamma ? xv * gamma[32 * b + lane] : xv;
    float a = fabsf(v);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
    const float dd = a / 127.0f;
    const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
    float r = roundf(v * id);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    const int qi = static_cast<int>(r);
    q[m * K + 32 * b + lane] = static_cast<int8_t>(qi);
    int s = qi;
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 32);
    float sq = xv * xv;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 32);
    if ((lane & 15) == 0) s16[m * (K / 16) + 2 * b + (lane >> 4)] = s;
    if (lane == 0) {
        d[m * nb + b] = dd;
        if (sumsq) sumsq[m * nb + b] = sq;
    }
}

}  // namespace sv

extern "C" int sv_quantize_act_q8(const float *x, int32_t M, int64_t K, const float *gamma, int8_t *q, float *d,
                                  int32_t *s16, float *sumsq, void *stream) {
    SV_REQUIRE(x && q && d && s16, SV_ERR_ARG, "quantize_act_q8: NULL buffer");
    SV_REQUIRE(M >= 1 && M <= SV_MAX_M, SV_ERR_ARG, "quantize_act_q8: M must be in [1, 16]");
    SV_REQUIRE(K > 0 && K % 32 == 0, SV_ERR_SHAPE, "quantize_act_q8: K must be a positive multiple of 32");
    SV_REQUIRE(sv::aligned(x, 4) && sv::aligned(d, 4) && sv::aligned(s16, 4) && (!gamma || sv::aligned(gamma, 4)) &&
                   (!sumsq || sv::aligned(sumsq, 4)),
               SV_ERR_ALIGN, "quantize_act_q8: fp32/int32 buffers must be 4-byte aligned");
    const int64_t items = static_cast<int64_t>(M) * (K / 32);
    const int64_t blocks = (items + 7) / 8;
    SV_REQUIRE(blocks < (1ll << 31), SV_ERR_SHAPE, "quantize_act_q8: too large");
    hipLaunchKernelGGL(sv::quant_act_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       sv::as_stream(stream), x, gamma, M, K, q, d, s16, sumsq);
    return sv::hip_check(hipGetLastError(), "quantize_act_q8 launch");
}
