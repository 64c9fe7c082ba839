// Host-side launchers shared between the translation units of the library.
#pragma once

#include <hip/hip_runtime.h>

#include "ql_common.hpp"

namespace ql {

hipError_t launch_pack(const Layout &L, const void *codes, const void *scales, const void *aux_in,
                       void *pw, void *ps, void *paux, hipStream_t st);
hipError_t launch_unpack(const Layout &L, const void *pw, const void *ps, const void *paux,
                         void *codes, void *scales, void *aux_out, hipStream_t st);
hipError_t launch_dequant_tile(const Layout &L, const void *pw, const void *ps, const void *paux, int64_t n0,
                               int64_t k0, int64_t tn, int64_t tk, int mode, float *out, hipStream_t st);

hipError_t launch_quantize(int fmt, int64_t N, int64_t K, int group, bool zp, const float *w,
                           const float *levels_host, void *codes, void *scales, void *zeros, hipStream_t st);
hipError_t launch_quant_act(const uint16_t *x, int M, int K, int Kp, int layout, int8_t *codes, float *scales,
                            hipStream_t st);
hipError_t launch_gemm_a8(const Layout &L, int tile, const uint16_t *x, int M, const void *pw, const void *ps,
                          const void *bias, void *out, bool out_f32, int8_t *xq, float *xs, hipStream_t st);
hipError_t launch_lora_merge8(const Layout &L, void *pw, void *ps, const void *mat1, const void *mat2, int rank,
                              float alpha, float beta, int stochastic, uint64_t seed, hipStream_t st);

// One translation unit per format family keeps the template instantiations apart.
hipError_t launch_gemm_int4(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_int4_zp(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_int8(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_mxfp4(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_cb4(const Layout &L, const Plan &p, const GemmArgs &a, hipStream_t st);
hipError_t launch_reduce(const GemmArgs &a, hipStream_t st);
hipError_t launch_swiglu(const uint16_t *x, uint16_t *h, int M, int K, hipStream_t st);
hipError_t launch_moe_plan(const int32_t *counts, int E, int T, int rows, int slots, int *offsets, int *tile_map,
                           hipStream_t st);

}  // namespace ql
