// INT4 instantiations of the linear kernel: symmetric weights here, weights with
// zero-points in ql_gemm_int4_zp.hip (two units, so they compile in parallel).
#include "ql_gemm_dispatch.hpp"
#include "ql_launch.hpp"

namespace ql {
hipError_t launch_gemm_int4(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st) {
    return L.zeros ? launch_gemm_int4_zp(L, p, a, st) : launch_qmm_group<FMT_INT4, false>(L, p, a, st);
}
}  // namespace ql
