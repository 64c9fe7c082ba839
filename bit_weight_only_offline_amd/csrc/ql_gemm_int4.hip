// INT4 (symmetric and with zero-points) instantiations of the linear kernel.
#include "ql_gemm_dispatch.hpp"
#include "ql_launch.hpp"

namespace ql {
hipError_t launch_gemm_int4(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st) {
    return L.zeros ? launch_qmm_group<FMT_INT4, true>(L, p, a, st) : launch_qmm_group<FMT_INT4, false>(L, p, a, st);
}
}  // namespace ql
