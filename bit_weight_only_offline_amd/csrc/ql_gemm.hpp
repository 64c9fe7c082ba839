// The weight-only linear kernel: Y = A . D(Wq)^T + b on gfx950 matrix cores.
//
// Workgroup = 4 wavefronts side by side along N, all walking the same k-range
// [kc0, kc0 + cps) chunk by chunk:
//   * the activation rows of the workgroup (16*MT of them) are staged through LDS,
//     double buffered, one chunk ahead, in the A-fragment order of
//     v_mfma_f32_16x16x32_bf16 (the SwiGLU input stage h = up * silu(gate) runs here,
//     once per workgroup and chunk);
//   * every wavefront streams its own NT column tiles straight from HBM into registers
//     with ranged dwordx4 buffer loads, PF chunks ahead, decodes them in registers
//     (ql_decode.hpp) and issues MT x NT MFMAs per 32-wide k-step;
//   * INT4/INT8 operands are offset by a constant (128+u or u), so each group's
//     partial sum is corrected with the group's row sums of A, computed by one more
//     MFMA against a ones operand, then scaled:  acc += s * (tmp - (128+z) * xsum);
//   * the epilogue applies the codebook row scale, adds the bias and rounds to bf16,
//     or, when the k-range is split over workgroups, stores float32 partial sums that
//     qreduce_kernel adds in a fixed order.
// Small M (decode) uses MT = 1 with deep prefetch and split-K across workgroups to keep
// every compute unit streaming; large M uses MT = 8 (128 rows) per workgroup.
#pragma once

#include <hip/hip_runtime.h>

#include "ql_common.hpp"
#include "ql_decode.hpp"

namespace ql {

__device__ inline uint32_t swiglu_pair(uint32_t up2, uint32_t gate2) {
    float h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float u = bf16_bits_to_f32((up2 >> (16 * e)) & 0xFFFFu);
        const float g = bf16_bits_to_f32((gate2 >> (16 * e)) & 0xFFFFu);
        h[e] = u * (g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)));
    }
    return pack_bf16x2(h[0], h[1]);
}

template <int FMT, bool ZP, int GS, int MT, int NT, int PF>
__global__ void __launch_bounds__(WG_THREADS) qmm_kernel(GemmArgs a) {
    constexpr int CH = chunk_k(FMT);
    constexpr int STEPS = CH / 32;
    constexpr int MP = 16 * MT;
    constexpr bool INTF = (FMT == FMT_INT4 || FMT == FMT_INT8);
    constexpr int SPC = INTF ? (GS <= STEPS ? STEPS / GS : 1) : 1;
    constexpr int STAGE = CH * MP * 2;
    constexpr int PIECES = MP * CH / 8;
    constexpr int PPT = (PIECES + WG_THREADS - 1) / WG_THREADS;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int ntb = (blockIdx.x * 4 + wv) * NT;
    const int m0 = blockIdx.y * MP;
    const int kz = blockIdx.z;
    const int kc0 = kz * a.cps;
    const int nck = min(a.kchunks - kc0, a.cps);

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, ZP ? a.z_bytes : 0u);

    CbLut lut = {0u, 0u, 0u, 0u};
    if (FMT == FMT_CB4) lut = reinterpret_cast<const CbRecord *>(a.aux)->lut;

    f32x4 acc[MT][NT];
    f32x4 tmp[MT][NT];
    f32x4 xs[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        xs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            tmp[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    u32x4 wreg[PF][NT];
    uint32_t sreg[PF][NT][SPC];
    uint32_t zreg[PF][NT][SPC];

    // ---- weight / scale prefetch of chunk i (relative to kc0) into slot u ----
    auto load_chunk = [&](int i, u32x4 (&wq)[NT], uint32_t (&sq)[NT][SPC], uint32_t (&zq)[NT][SPC]) {
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
                    sq[j][q] = ld16(sr, (rec * TILE_N + c) * 2);
                    if (ZP) zq[j][q] = ld8(zr, rec * 8 + (c >> 1));
                }
            }
        }
    };

    // ---- activation staging of chunk i: global -> registers -> LDS (A-fragment order) ----
    u32x4 ar[PPT], gr[PPT];
    auto stage_load = [&](int i) {
        const int kbase = (kc0 + i) * CH;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int piece = tid + WG_THREADS * p;
            ar[p] = u32x4{0u, 0u, 0u, 0u};
            gr[p] = u32x4{0u, 0u, 0u, 0u};
            if (PIECES % WG_THREADS == 0 || piece < PIECES) {
                const int r = piece / (CH / 8), q8 = piece % (CH / 8);
                const int m = m0 + r, k = kbase + q8 * 8;
                if (m < a.M && k < a.K) {
                    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.x + int64_t(m) * a.ldx + k);
                    ar[p] = *src;
                    if (a.swiglu) gr[p] = *reinterpret_cast<const u32x4 *>(a.x + int64_t(m) * a.ldx + a.K + k);
                }
            }
        }
    };
    auto stage_store = [&](int st) {
        uint8_t *base = lds + st * STAGE;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int piece = tid + WG_THREADS * p;
            if (PIECES % WG_THREADS == 0 || piece < PIECES) {
                const int r = piece / (CH / 8), q8 = piece % (CH / 8);
                const int t = q8 >> 2, gg = q8 & 3;
                u32x4 v = ar[p];
                if (a.swiglu) {
                    v.x = swiglu_pair(ar[p].x, gr[p].x);
                    v.y = swiglu_pair(ar[p].y, gr[p].y);
                    v.z = swiglu_pair(ar[p].z, gr[p].z);
                    v.w = swiglu_pair(ar[p].w, gr[p].w);
                }
                *reinterpret_cast<u32x4 *>(base + ((t * 4 + gg) * MP + r) * 16) = v;
            }
        }
    };

    const u32x4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 ones = as_bf16x8(ones_u);

    // ---- one chunk of MFMAs from LDS stage st and weight slot (wq, sq, zq) ----
    auto compute = [&](int i, int st, const u32x4 (&wq)[NT], const uint32_t (&sq)[NT][SPC],
                       const uint32_t (&zq)[NT][SPC]) {
        const int kc = kc0 + i;
        const uint8_t *base = lds + st * STAGE;
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            bf16x8 af[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[mt] = *reinterpret_cast<const bf16x8 *>(base + ((t * 4 + g) * MP + mt * 16 + c) * 16);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                u32x4 bw;
                if (FMT == FMT_INT4) bw = dec_int4(wq[j][t]);
                else if (FMT == FMT_INT8) bw = dec_int8(wq[j][2 * t], wq[j][2 * t + 1]);
                else if (FMT == FMT_MXFP4) bw = dec_mxfp4(wq[j][t], e8m0_to_f32((sq[j][0] >> (8 * t)) & 0xFFu));
                else bw = dec_cb4(wq[j][t], lut);
                const bf16x8 b = as_bf16x8(bw);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (INTF) tmp[mt][j] = mfma16x16x32(af[mt], b, tmp[mt][j]);
                    else acc[mt][j] = mfma16x16x32(af[mt], b, acc[mt][j]);
                }
            }
            if (INTF) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xs[mt] = mfma16x16x32(af[mt], ones, xs[mt]);
                bool boundary;
                if (GS <= STEPS) boundary = ((t + 1) % GS) == 0;
                else boundary = (t == STEPS - 1) && (((kc + 1) % (GS / STEPS)) == 0);
                if (boundary) {
                    const int q = (GS <= STEPS) ? (t / GS) : 0;
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        float s, off;
                        if (FMT == FMT_INT4) {
                            s = f16_bits_to_f32(sq[j][q]);
                            off = ZP ? 128.0f + float((zq[j][q] >> (4 * (c & 1))) & 0xFu) : 136.0f;
                        } else {
                            s = bf16_bits_to_f32(sq[j][q]);
                            off = 128.0f;
                        }
                        const float cz = -s * off;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                acc[mt][j][r] = fmaf(s, tmp[mt][j][r], acc[mt][j][r]);
                                acc[mt][j][r] = fmaf(cz, xs[mt][r], acc[mt][j][r]);
                            }
                            tmp[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) xs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };

    // ---- prologue ----
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (u < nck) load_chunk(u, wreg[u], sreg[u], zreg[u]);
    stage_load(0);
    stage_store(0);
    __syncthreads();

    // ---- main loop ----
    for (int i0 = 0; i0 < nck; i0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int i = i0 + u;
            if (i < nck) {
                const bool more = (i + 1) < nck;
                if (more) stage_load(i + 1);
                compute(i, i & 1, wreg[u], sreg[u], zreg[u]);
                if (i + PF < nck) load_chunk(i + PF, wreg[u], sreg[u], zreg[u]);
                if (more) stage_store((i + 1) & 1);
                __syncthreads();
            }
        }
    }

    // ---- epilogue ----
    float rs[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        rs[j] = 1.0f;
        if (FMT == FMT_CB4) {
            const int n = (ntb + j) * TILE_N + c;
            if (n < a.Np)
                rs[j] = reinterpret_cast<const float *>(a.s)[n] * reinterpret_cast<const CbRecord *>(a.aux)->inv_alpha;
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int n = (ntb + j) * TILE_N + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + mt * 16 + g * 4 + r;
                if (m >= a.M) continue;
                float v = acc[mt][j][r];
                if (a.ks == 1) {
                    if (n >= a.N) continue;
                    if (FMT == FMT_CB4) v *= rs[j];
                    if (a.bias) v += bf16_bits_to_f32(a.bias[n]);
                    if (a.out_f32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
                    else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
                } else if (n < a.Np) {
                    a.ws[(int64_t(kz) * a.M + m) * a.Np + n] = v;
                }
            }
        }
    }
}

}  // namespace ql
