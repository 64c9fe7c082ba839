// Small kernels around the linear: the split-K reduce of the tile schedules and the
// SwiGLU prologue of the decode schedules.
#include <hip/hip_runtime.h>

#include "ql_common.hpp"
#include "ql_decode.hpp"
#include "ql_gemm.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

// Adds the ks float32 partial sums of each output in split order (s = 0, 1, ...),
// then applies the epilogue.
__global__ void __launch_bounds__(256) qreduce_kernel(GemmArgs a) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= int64_t(a.M) * a.N) return;
    const int m = int(idx / a.N), n = int(idx % a.N);
    float v = 0.0f;
    for (int s = 0; s < a.ks; ++s) v += a.ws[(int64_t(s) * a.M + m) * a.Np + n];
    if (a.aux) v *= reinterpret_cast<const float *>(a.s)[n] * reinterpret_cast<const CbRecord *>(a.aux)->inv_alpha;
    if (a.bias) v += bf16_bits_to_f32(a.bias[n]);
    if (a.out_f32) reinterpret_cast<float *>(a.out)[idx] = v;
    else reinterpret_cast<__bf16 *>(a.out)[idx] = (__bf16)v;
}

// h = bf16(up * silu(gate)) for a raw [M, 2K] input, 8 inputs per thread (the same
// arithmetic as the fused staging of the tile kernels).
__global__ void __launch_bounds__(256) swiglu_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ h,
                                                     int M, int K) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;   // index of an 8-wide piece
    const int per_row = K / 8;
    if (i >= int64_t(M) * per_row) return;
    const int m = int(i / per_row), k = int(i % per_row) * 8;
    const u32x4 up = *reinterpret_cast<const u32x4 *>(x + int64_t(m) * 2 * K + k);
    const u32x4 gt = *reinterpret_cast<const u32x4 *>(x + int64_t(m) * 2 * K + K + k);
    u32x4 o;
    o.x = swiglu_pair(up.x, gt.x);
    o.y = swiglu_pair(up.y, gt.y);
    o.z = swiglu_pair(up.z, gt.z);
    o.w = swiglu_pair(up.w, gt.w);
    *reinterpret_cast<u32x4 *>(h + int64_t(m) * K + k) = o;
}

}  // namespace

hipError_t launch_reduce(const GemmArgs &a, hipStream_t st) {
    const int64_t n = int64_t(a.M) * a.N;
    hipLaunchKernelGGL(qreduce_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t *x, uint16_t *h, int M, int K, hipStream_t st) {
    const int64_t n = int64_t(M) * (K / 8);
    hipLaunchKernelGGL(swiglu_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, x, h, M, K);
    return hipGetLastError();
}

// Grouped launch plan: expert offsets (exclusive prefix sum of the token counts, each
// count clamped to [0, tokens left] so rows never run past T) and the slot map, expert
// by expert in order, unused slots marked -1.  One thread: E and the slot count are small
// and the order is then fixed.
__global__ void moe_plan_kernel(const int32_t *__restrict__ counts, int E, int T, int rows, int slots,
                                int *__restrict__ offsets, int *__restrict__ tile_map) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int run = 0, t = 0;
    for (int e = 0; e < E; ++e) {
        const int c = min(max(counts[e], 0), T - run);
        offsets[e] = run;
        for (int r = 0; r < c && t < slots; r += rows, ++t) {
            tile_map[2 * t] = e;
            tile_map[2 * t + 1] = r;
        }
        run += c;
    }
    offsets[E] = run;
    for (; t < slots; ++t) {
        tile_map[2 * t] = -1;
        tile_map[2 * t + 1] = 0;
    }
}

hipError_t launch_moe_plan(const int32_t *counts, int E, int T, int rows, int slots, int *offsets, int *tile_map,
                           hipStream_t st) {
    hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(64), 0, st, counts, E, T, rows, slots, offsets, tile_map);
    return hipGetLastError();
}

}  // namespace ql
