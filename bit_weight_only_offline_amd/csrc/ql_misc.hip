// Small kernels around the linear: the split-K reduce of the tile schedules and the
// SwiGLU prologue that materialises h when the linear kernel does not form it itself.
#include <hip/hip_runtime.h>

#include "ql_common.hpp"
#include "ql_decode.hpp"
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

// Mixture-of-experts plan: expert offsets (the running sum of the counts, each count
// clamped to [0, tokens left] so rows never run past T) and the slot map, expert by
// expert in order, unused slots marked -1.  One workgroup: block-wide prefix sums of the
// clamped counts and of each expert's number of row blocks, 256 experts at a time; each
// expert's thread writes its own slots.  The result is the same as walking the experts
// one by one.
__global__ void __launch_bounds__(256) moe_plan_kernel(const int32_t *__restrict__ counts, int E, int T, int rows,
                                                       int slots, int *__restrict__ offsets,
                                                       int *__restrict__ tile_map) {
    __shared__ int64_t tok[256];
    __shared__ int blk[256];
    const int t = threadIdx.x;
    int64_t run = 0;                 // clamped tokens of the experts before this batch
    int used = 0;                    // slots taken by them
    for (int e0 = 0; e0 < E; e0 += 256) {
        const int e = e0 + t;
        const int own = e < E ? min(max(counts[e], 0), T) : 0;
        tok[t] = own;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {               // inclusive scan of the counts
            const int64_t v = t >= d ? tok[t - d] : 0;
            __syncthreads();
            tok[t] += v;
            __syncthreads();
        }
        const int64_t incl = tok[t], batch = tok[255];
        const int start = int(min(run + incl - own, int64_t(T)));
        const int end = int(min(run + incl, int64_t(T)));
        const int c = end - start;
        const int nb = (c + rows - 1) / rows;
        __syncthreads();
        blk[t] = nb;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {               // inclusive scan of the row blocks
            const int v = t >= d ? blk[t - d] : 0;
            __syncthreads();
            blk[t] += v;
            __syncthreads();
        }
        const int first = used + blk[t] - nb;
        if (e < E) {
            offsets[e] = start;
            for (int r = 0; r < nb && first + r < slots; ++r) {
                tile_map[2 * (first + r)] = e;
                tile_map[2 * (first + r) + 1] = r * rows;
            }
        }
        used += blk[255];
        run = min(run + batch, int64_t(T));
        __syncthreads();                                  // before the next batch reuses LDS
    }
    if (t == 0) offsets[E] = int(run);
    for (int k = min(used, slots) + t; k < slots; k += 256) {
        tile_map[2 * k] = -1;
        tile_map[2 * k + 1] = 0;
    }
}

hipError_t launch_moe_plan(const int32_t *counts, int E, int T, int rows, int slots, int *offsets, int *tile_map,
                           hipStream_t st) {
    hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(256), 0, st, counts, E, T, rows, slots, offsets, tile_map);
    return hipGetLastError();
}

}  // namespace ql
