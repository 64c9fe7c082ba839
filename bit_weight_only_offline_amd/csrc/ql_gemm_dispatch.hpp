// Selects the compiled tile shape of the linear kernel for one format.
#pragma once

#include <type_traits>

#include "ql_gemv.hpp"
#include "ql_gemm_lds.hpp"

namespace ql {

// Raise a kernel's dynamic-LDS limit to `bytes`, once per kernel (the flag is per
// instantiation of the caller).
inline hipError_t allow_dynamic_lds(const void *kern, size_t bytes, bool &done) {
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e == hipSuccess) done = true;
    return e;
}

template <int FMT, bool ZP, int GS, int I>
hipError_t launch_one(const Plan &p, const GemmArgs &a, hipStream_t st) {
    constexpr TileCfg t = TILE_CFGS[I];
    if constexpr (t.kind == 0) {
        auto go = [&](auto sw, auto x1) {
            constexpr bool SW = decltype(sw)::value, X1 = decltype(x1)::value;
            auto kern = qgemv_kernel<FMT, ZP, GS, t.NT, t.WK, t.PF, SW, X1>;
            constexpr size_t lds = gemv_lds_bytes(FMT, ZP, GS, t.NT, t.WK, t.PF, SW, X1);
            static bool attr_set = false;
            hipError_t e = allow_dynamic_lds((const void *)kern, lds, attr_set);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kern, dim3(p.nblocks, a.tile_map ? a.slots : 1), dim3(64 * t.WK), lds, st, a);
            return hipSuccess;
        };
        hipError_t e = p.fuse_swiglu ? go(std::true_type{}, std::false_type{})
                       : (p.x1 ? go(std::false_type{}, std::true_type{}) : go(std::false_type{}, std::false_type{}));
        if (e != hipSuccess) return e;
    } else {
        static_assert(t.kind == 2, "decode or LDS-ring schedule");
        constexpr int wk = ring_wk(FMT, t.WK);
        // chunks per ring stage: two for chunk-parallel schedules where two such stages fit
        constexpr int cs = t.CP && 4 * ring_stage_bytes(FMT, ZP, GS, t.WM, t.WN, wk, t.MT, t.NT) <= LDS_BYTES_MAX ? 2 : 1;
        constexpr int depth = ring_depth(FMT, ZP, GS, t.WM, t.WN, wk, t.MT, t.NT, t.PF, cs);
        constexpr size_t lds = ring_lds_bytes(FMT, ZP, GS, t.WM, t.WN, wk, t.MT, t.NT, depth, cs);
        auto kern = qgemm_lds_kernel<FMT, ZP, GS, t.WM, t.WN, wk, t.MT, t.NT, depth, cs == 2>;
        static_assert(lds <= LDS_BYTES_MAX, "ring fits the LDS");
        static bool attr_set = false;
        hipError_t e = allow_dynamic_lds((const void *)kern, lds, attr_set);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(p.mtiles * p.nblocks, p.ks), dim3(64 * t.WM * t.WN * wk), lds, st, a);
    }
    return hipGetLastError();
}

template <int FMT, bool ZP, int GS>
hipError_t launch_qmm_cfg(const Plan &p, const GemmArgs &a, hipStream_t st) {
    static_assert(NUM_TILE_CFGS == 25, "one case per compiled schedule");
    switch (p.cfg) {
        case 0: return launch_one<FMT, ZP, GS, 0>(p, a, st);
        case 1: return launch_one<FMT, ZP, GS, 1>(p, a, st);
        case 2: return launch_one<FMT, ZP, GS, 2>(p, a, st);
        case 3: return launch_one<FMT, ZP, GS, 3>(p, a, st);
        case 4: return launch_one<FMT, ZP, GS, 4>(p, a, st);
        case 5: return launch_one<FMT, ZP, GS, 5>(p, a, st);
        case 6: return launch_one<FMT, ZP, GS, 6>(p, a, st);
        case 7: return launch_one<FMT, ZP, GS, 7>(p, a, st);
        case 8: return launch_one<FMT, ZP, GS, 8>(p, a, st);
        case 9: return launch_one<FMT, ZP, GS, 9>(p, a, st);
        case 10: return launch_one<FMT, ZP, GS, 10>(p, a, st);
        case 11: return launch_one<FMT, ZP, GS, 11>(p, a, st);
        case 12: return launch_one<FMT, ZP, GS, 12>(p, a, st);
        case 13: return launch_one<FMT, ZP, GS, 13>(p, a, st);
        case 14: return launch_one<FMT, ZP, GS, 14>(p, a, st);
        case 15: return launch_one<FMT, ZP, GS, 15>(p, a, st);
        case 16: return launch_one<FMT, ZP, GS, 16>(p, a, st);
        case 17: return launch_one<FMT, ZP, GS, 17>(p, a, st);
        case 18: return launch_one<FMT, ZP, GS, 18>(p, a, st);
        case 19: return launch_one<FMT, ZP, GS, 19>(p, a, st);
        case 20: return launch_one<FMT, ZP, GS, 20>(p, a, st);
        case 21: return launch_one<FMT, ZP, GS, 21>(p, a, st);
        case 22: return launch_one<FMT, ZP, GS, 22>(p, a, st);
        case 23: return launch_one<FMT, ZP, GS, 23>(p, a, st);
        case 24: return launch_one<FMT, ZP, GS, 24>(p, a, st);
        default: return hipErrorInvalidValue;
    }
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
