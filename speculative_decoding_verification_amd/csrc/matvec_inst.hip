// matvec_inst.hip - the projection and pass kernels for one number of
// positions.  The build compiles this file once per M in 1..16 with
// -DSV_INST_M=<M>, so the sixteen kernel variants build in parallel; the
// host side (matvec.hip) reaches them through the templates declared in
// matvec_launch.h.
#include "matvec_dev.h"

#ifndef SV_INST_M
#error "compile with -DSV_INST_M=<positions>"
#endif

namespace sv {

template <>
void launch_pass_m<SV_INST_M>(int grid, size_t lds, hipStream_t st, const PhaseDesc *table, int n_phases,
                              const uint32_t *sched, unsigned *ctl, int CS, ArgmaxList am,
                              unsigned long long *trace) {
    hipLaunchKernelGGL((pass_kernel<SV_INST_M>), dim3(grid), dim3(kThreads), lds, st, table, n_phases, sched, ctl, CS,
                       am, trace);
}

template <>
void launch_phase_m<SV_INST_M>(int grid, size_t lds, hipStream_t st, const PhaseDesc &P, int CS) {
    hipLaunchKernelGGL((phase_kernel<SV_INST_M>), dim3(grid), dim3(kThreads), lds, st, P);
}

template <>
int occupancy_pass_m<SV_INST_M>(size_t lds) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(&pass_kernel<SV_INST_M>),
                                                     kThreads, lds) != hipSuccess)
        return 0;
    return n;
}

// Dynamic LDS above the default 64 KiB must be allowed per kernel.
template <>
hipError_t allow_lds_m<SV_INST_M>(size_t lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&pass_kernel<SV_INST_M>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&phase_kernel<SV_INST_M>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}

template <>
hipError_t pass_attr_m<SV_INST_M>(hipFuncAttributes *fa) {
    return hipFuncGetAttributes(fa, reinterpret_cast<const void *>(&pass_kernel<SV_INST_M>));
}

}  // namespace sv
