// Decode-shape kernel (M <= 16): split-K within the workgroup, wavefront-reduced.
//
// One workgroup owns NT column tiles (16*NT output columns) over the whole input
// dimension; its WK wavefronts split the chunks of the input dimension into WK
// contiguous runs (whole groups each).  Every wavefront streams its run of packed
// weight tiles and the matching A fragments (the activation rows, read straight into
// registers) PF chunks ahead, decodes the weights in registers and accumulates with
// v_mfma_f32_16x16x32_bf16 (A rows beyond M are never loaded: their products only
// reach output rows that are not stored).  At the end the WK partial tiles are added in
// LDS in wavefront order -- a fixed order -- and the epilogue applies the codebook row
// scale and the bias and rounds to bf16.  No workspace, no cross-workgroup traffic.
#pragma once

#include <hip/hip_runtime.h>

#include "ql_common.hpp"
#include "ql_decode.hpp"

namespace ql {

template <int FMT, bool ZP, int GS, int NT, int WK, int PF>
__global__ void __launch_bounds__(64 * WK) qgemv_kernel(GemmArgs a) {
    constexpr int CH = chunk_k(FMT);
    constexpr int STEPS = CH / 32;
    constexpr bool INTF = (FMT == FMT_INT4 || FMT == FMT_INT8);
    constexpr int SPC = INTF ? (GS <= STEPS ? STEPS / GS : 1) : 1;
    __shared__ float red[WK][NT][4][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keep it scalar
    const int g = lane >> 4, c = lane & 15;
    const int ntb = blockIdx.x * NT;
    // this wavefront's run of chunks: cps per wavefront (a multiple of the group span)
    const int kc0 = wv * a.cps;
    const int nck = max(0, min(a.kchunks - kc0, a.cps));

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, ZP ? a.z_bytes : 0u);
    const uint32_t s_shift = 16u * (c & 1);                       // this column's fp16/bf16 scale
    const uint32_t z_shift = 8u * ((c >> 1) & 3) + 4u * (c & 1);  // and its 4-bit zero-point

    CbLut lut = {0u, 0u, 0u, 0u};
    if (FMT == FMT_CB4) lut = reinterpret_cast<const CbRecord *>(a.aux)->lut;

    f32x4 acc[NT], tmp[NT], xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        tmp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    u32x4 wreg[PF][NT];
    uint32_t sreg[PF][NT][SPC];
    uint32_t zreg[PF][NT][SPC];
    u32x4 xreg[PF][STEPS];
    // activations through a ranged buffer: rows >= M and inputs >= K read as zero
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint32_t(int64_t(a.M) * a.ldx * 2));
    // lanes of rows >= M read from an offset beyond the buffer (bit 31 set)
    const uint32_t xrow = (c < a.M) ? uint32_t(c) * uint32_t(a.ldx) * 2u : 0x80000000u;

    auto load_chunk = [&](int i, u32x4 (&wq)[NT], uint32_t (&sq)[NT][SPC], uint32_t (&zq)[NT][SPC],
                          u32x4 (&xq)[STEPS]) {
        const int kc = kc0 + i;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const uint32_t tile = uint32_t(ntb + j) * uint32_t(a.kchunks) + uint32_t(kc);
            wq[j] = ld128(wr, tile * TILE_BYTES + lane * 16);
            if (FMT == FMT_MXFP4) {
                sq[j][0] = ld32(sr, (tile * TILE_N + c) * 4);
            } else if (INTF) {
#pragma unroll
                for (int q = 0; q < SPC; ++q) {
                    const uint32_t grp = (GS <= STEPS) ? uint32_t(kc * (STEPS / GS) + q) : uint32_t(kc / (GS / STEPS));
                    const uint32_t rec = uint32_t(ntb + j) * uint32_t(a.ngroups) + grp;
                    // aligned 32-bit words; the lane's field is selected when it is used,
                    // so no extension of a sub-dword load forces an early wait
                    sq[j][q] = ld32(sr, ((rec * TILE_N + c) * 2) & ~3u);
                    if (ZP) zq[j][q] = ld32(zr, (rec * 8 + (c >> 1)) & ~3u);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const int k = kc * CH + 32 * t + 8 * g;
            const uint32_t past_k = uint32_t(~(int32_t(k - a.K) >> 31)) & 0x80000000u;   // k >= K
            xq[t] = ld128(xr, (xrow + uint32_t(k) * 2u) | past_k);
        }
    };

    const u32x4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 ones = as_bf16x8(ones_u);

    auto compute = [&](int i, const u32x4 (&wq)[NT], const uint32_t (&sq)[NT][SPC], const uint32_t (&zq)[NT][SPC],
                       const u32x4 (&xq)[STEPS]) {
        const int kc = kc0 + i;
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const bf16x8 af = as_bf16x8(xq[t]);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                u32x4 bw;
                if (FMT == FMT_INT4) bw = dec_int4(wq[j][t]);
                else if (FMT == FMT_INT8) bw = dec_int8(wq[j][2 * t], wq[j][2 * t + 1]);
                else if (FMT == FMT_MXFP4) bw = dec_mxfp4(wq[j][t], e8m0_to_f32((sq[j][0] >> (8 * t)) & 0xFFu));
                else bw = dec_cb4(wq[j][t], lut);
                if (INTF) tmp[j] = mfma16x16x32(af, as_bf16x8(bw), tmp[j]);
                else acc[j] = mfma16x16x32(af, as_bf16x8(bw), acc[j]);
            }
            if (INTF) {
                xs = mfma16x16x32(af, ones, xs);
                bool boundary;
                if (GS <= STEPS) boundary = ((t + 1) % GS) == 0;
                else boundary = (t == STEPS - 1) && (((kc + 1) % (GS / STEPS)) == 0);
                if (boundary) {
                    const int q = (GS <= STEPS) ? (t / GS) : 0;
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        float s, off;
                        const uint32_t sbits = (sq[j][q] >> s_shift) & 0xFFFFu;
                        if (FMT == FMT_INT4) {
                            s = f16_bits_to_f32(sbits);
                            off = ZP ? 128.0f + float((zq[j][q] >> z_shift) & 0xFu) : 136.0f;
                        } else {
                            s = bf16_bits_to_f32(sbits);
                            off = 128.0f;
                        }
                        const float cz = -s * off;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            acc[j][r] = fmaf(s, tmp[j][r], acc[j][r]);
                            acc[j][r] = fmaf(cz, xs[r], acc[j][r]);
                        }
                        tmp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                    xs = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };

#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (u < nck) load_chunk(u, wreg[u], sreg[u], zreg[u], xreg[u]);
    for (int i0 = 0; i0 < nck; i0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int i = i0 + u;
            if (i < nck) {
                compute(i, wreg[u], sreg[u], zreg[u], xreg[u]);
                if (i + PF < nck) load_chunk(i + PF, wreg[u], sreg[u], zreg[u], xreg[u]);
            }
        }
    }

    // ---- wavefront reduction in LDS (fixed order), then the epilogue ----
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wv][j][r][lane] = acc[j][r];
    __syncthreads();
    // output element e = (j, r, lane): row g*4 + r, column (ntb + j)*16 + c
    for (int e = tid; e < NT * 4 * 64; e += 64 * WK) {
        const int j = e / 256, r = (e / 64) % 4, l = e % 64;
        const int m = (l >> 4) * 4 + r, n = (ntb + j) * TILE_N + (l & 15);
        if (m >= a.M || n >= a.N) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WK; ++w) v += red[w][j][r][l];
        if (FMT == FMT_CB4) v *= reinterpret_cast<const float *>(a.s)[n] * reinterpret_cast<const CbRecord *>(a.aux)->inv_alpha;
        if (a.bias) v += bf16_bits_to_f32(a.bias[n]);
        if (a.out_f32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
        else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
    }
}

}  // namespace ql
