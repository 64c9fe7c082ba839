// INT4 with zero-points: instantiations of the linear kernel.
#include "ql_gemm_dispatch.hpp"
#include "ql_launch.hpp"

namespace ql {
hipError_t launch_gemm_int4_zp(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st) {
    return launch_qmm_group<FMT_INT4, true>(L, p, a, st);
}
}  // namespace ql
