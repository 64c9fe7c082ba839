// Selects the compiled tile shape of the linear kernel for one format.
#pragma once

#include "ql_gemm.hpp"

namespace ql {

template <int FMT, bool ZP, int GS>
hipError_t launch_qmm_cfg(const Plan &p, const GemmArgs &a, hipStream_t st) {
    const dim3 grid(p.nblocks, p.mtiles, p.ks), block(WG_THREADS);
    switch (p.cfg) {
        case 0: hipLaunchKernelGGL((qmm_kernel<FMT, ZP, GS, 1, 1, 8>), grid, block, 0, st, a); break;
        case 1: hipLaunchKernelGGL((qmm_kernel<FMT, ZP, GS, 1, 2, 4>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((qmm_kernel<FMT, ZP, GS, 2, 2, 4>), grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL((qmm_kernel<FMT, ZP, GS, 4, 2, 4>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((qmm_kernel<FMT, ZP, GS, 8, 2, 2>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

template <int FMT, bool ZP>
hipError_t launch_qmm_group(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st) {
    switch (L.group) {
        case 32: return launch_qmm_cfg<FMT, ZP, 1>(p, a, st);
        case 64: return launch_qmm_cfg<FMT, ZP, 2>(p, a, st);
        case 128: return launch_qmm_cfg<FMT, ZP, 4>(p, a, st);
        default: return launch_qmm_cfg<FMT, ZP, 8>(p, a, st);
    }
}

}  // namespace ql
