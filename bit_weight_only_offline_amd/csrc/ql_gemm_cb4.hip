// 4-bit codebook instantiations of the linear kernel.
#include "ql_gemm_dispatch.hpp"
#include "ql_launch.hpp"

namespace ql {
hipError_t launch_gemm_cb4(const Layout &, const Plan &p, const GemmArgs &a, hipStream_t st) {
    return launch_qmm_cfg<FMT_CB4, false, 1>(p, a, st);
}
}  // namespace ql
