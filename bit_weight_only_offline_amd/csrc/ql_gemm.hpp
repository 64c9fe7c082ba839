// The weight-only linear kernel: Y = A . D(Wq)^T + b on gfx950 matrix cores.
//
// Workgroup = 4 wavefronts side by side along N, all walking the same k-range of the
// workgroup's split, stage by stage:
//   * the activation rows of the workgroup (16*MT of them) are staged through LDS in
//     blocks of SK inputs, double buffered: the global loads of block s+1 are in flight
//     while block s is consumed, and there is one barrier per block.  The layout in LDS
//     is the A-fragment order of v_mfma_f32_16x16x32_bf16, so every fragment read is one
//     conflict-free ds_read_b128.  The SwiGLU input stage h = up * silu(gate) runs here,
//     once per workgroup and block;
//   * every wavefront streams its own NT column tiles straight from HBM into registers
//     with ranged dwordx4 buffer loads, PF chunks ahead, decodes them in registers
//     (ql_decode.hpp) and issues MT x NT MFMAs per 32-wide k-step;
//   * INT4/INT8 operands carry a constant offset (128+u or u), so each group's partial
//     sum is corrected with the group's row sums of A, computed by one more MFMA against
//     a ones operand, and scaled:  acc += s * tmp - s * (128+z) * xsum;
//   * the epilogue applies the codebook row scale, adds the bias and rounds to bf16.
//     When the k-range is split over workgroups, each one stores float32 partial sums
//     instead and a reduce kernel adds them in split order (a fixed order, so results
//     do not depend on timing) and runs the epilogue.  Agent-scope fences for an
//     in-kernel reduction write back and invalidate each XCD's L2, which costs far more
//     than the second launch.
#pragma once

#include <hip/hip_runtime.h>

#include "ql_common.hpp"
#include "ql_decode.hpp"

namespace ql {

__device__ inline float epilogue_value(const GemmArgs &a, float v, int n, float rs) {
    if (a.aux) v *= rs;
    if (a.bias) v += bf16_bits_to_f32(a.bias[n]);
    return v;
}

__device__ inline void store_out(const GemmArgs &a, int m, int n, float v) {
    if (a.out_f32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
    else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
}

template <int FMT, bool ZP, int GS, int MT, int NT, int SK, int PF, bool SW>
__global__ void __launch_bounds__(WG_THREADS) qmm_kernel(GemmArgs a) {
    constexpr int CH = chunk_k(FMT);
    constexpr int STEPS = CH / 32;
    constexpr int SC = SK / CH;                     // chunks per LDS block
    constexpr int MP = 16 * MT;
    constexpr bool INTF = (FMT == FMT_INT4 || FMT == FMT_INT8);
    constexpr int SPC = INTF ? (GS <= STEPS ? STEPS / GS : 1) : 1;
    constexpr int STAGE = SK * MP * 2;
    constexpr int PIECES = MP * SK / 8;
    constexpr int PPT = (PIECES + WG_THREADS - 1) / WG_THREADS;
    constexpr int R = PF >= SC ? PF / SC : 1;       // LDS blocks per prefetch round
    static_assert(SK % CH == 0, "block must hold whole chunks");
    static_assert((PF % SC == 0) || (SC % PF == 0), "prefetch depth and block must nest");
    static_assert(2 * STAGE <= 65536, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keep it scalar
    const int g = lane >> 4, c = lane & 15;
    const int ntb = (blockIdx.x * 4 + wv) * NT;
    const int m0 = blockIdx.y * MP;
    const int kz = blockIdx.z;
    const int kc0 = kz * a.cps;
    const int nck = min(a.kchunks - kc0, a.cps);
    const int nst = (nck + SC - 1) / SC;

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, ZP ? a.z_bytes : 0u);
    const uint32_t s_shift = 16u * (c & 1);                       // this column's fp16/bf16 scale
    const uint32_t z_shift = 8u * ((c >> 1) & 3) + 4u * (c & 1);  // and its 4-bit zero-point

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

    // ---- weight / scale prefetch of chunk i (relative to kc0) into one slot ----
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
                    // aligned 32-bit words; the lane's field is selected when it is used,
                    // so no extension of a sub-dword load forces an early wait
                    sq[j][q] = ld32(sr, ((rec * TILE_N + c) * 2) & ~3u);
                    if (ZP) zq[j][q] = ld32(zr, (rec * 8 + (c >> 1)) & ~3u);
                }
            }
        }
    };

    // ---- activation block st (SK inputs): global -> registers -> LDS ----
    // Ranged buffer loads with branch-free offsets: rows >= M and inputs past the
    // split read as zero (offset with bit 31 set, beyond the buffer).
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint32_t(int64_t(a.M) * a.ldx * 2));
    u32x4 ar[PPT], gr[SW ? PPT : 1];
    auto stage_load = [&](int st) {
        const int kbase = (kc0 + st * SC) * CH;
        const int kend = min(a.K, (kc0 + nck) * CH);
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int piece = tid + WG_THREADS * p;
            const int r = piece / (SK / 8), q8 = piece % (SK / 8);
            const int m = m0 + r, k = kbase + q8 * 8;
            const uint32_t bad = (uint32_t(~(int32_t(k - kend) >> 31)) | uint32_t(~(int32_t(m - a.M) >> 31))) &
                                 0x80000000u;
            const uint32_t off = ((uint32_t(m) * uint32_t(a.ldx) + uint32_t(k)) * 2u) | bad;
            ar[p] = ld128(xr, off);
            if (SW) gr[SW ? p : 0] = ld128(xr, (off + uint32_t(a.K) * 2u) | bad);
        }
    };
    auto stage_store = [&](int buf) {
        uint8_t *base = lds + buf * STAGE;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int piece = tid + WG_THREADS * p;
            if (PIECES % WG_THREADS == 0 || piece < PIECES) {
                const int r = piece / (SK / 8), q8 = piece % (SK / 8);
                const int ks = q8 >> 2, gg = q8 & 3;   // k-step inside the block, 8-wide slice
                u32x4 v = ar[p];
                if (SW) {
                    const u32x4 gv = gr[SW ? p : 0];
                    v.x = swiglu_pair(v.x, gv.x);
                    v.y = swiglu_pair(v.y, gv.y);
                    v.z = swiglu_pair(v.z, gv.z);
                    v.w = swiglu_pair(v.w, gv.w);
                }
                *reinterpret_cast<u32x4 *>(base + ((ks * 4 + gg) * MP + r) * 16) = v;
            }
        }
    };

    const u32x4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 ones = as_bf16x8(ones_u);

    // ---- one chunk of MFMAs: chunk i, LDS block buf, position cc inside the block ----
    auto compute = [&](int i, int buf, int cc, const u32x4 (&wq)[NT], const uint32_t (&sq)[NT][SPC],
                       const uint32_t (&zq)[NT][SPC]) {
        const int kc = kc0 + i;
        const uint8_t *base = lds + buf * STAGE;
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const int ksb = cc * STEPS + t;          // k-step inside the LDS block
            bf16x8 af[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[mt] = *reinterpret_cast<const bf16x8 *>(base + ((ksb * 4 + g) * MP + mt * 16 + c) * 16);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                u32x4 bw;
                if (FMT == FMT_INT4) bw = dec_int4(wq[j][t]);
                else if (FMT == FMT_INT8) bw = dec_int8<true>(wq[j][2 * t], wq[j][2 * t + 1]);
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
                for (int mt = 0; mt < MT; ++mt)
                    if (FMT == FMT_INT4) xs[mt] = mfma16x16x32(af[mt], ones, xs[mt]);   // INT8 codes are signed
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
                            off = 0.0f;                   // the operand is the signed code
                        }
                        const float cz = -s * off;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                acc[mt][j][r] = fmaf(s, tmp[mt][j][r], acc[mt][j][r]);
                                if (FMT == FMT_INT4) acc[mt][j][r] = fmaf(cz, xs[mt][r], acc[mt][j][r]);
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

    // ---- main loop: rounds of R blocks x SC chunks = max(PF, SC) chunks ----
    for (int st0 = 0; st0 < nst; st0 += R) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int st = st0 + rr;
            if (st < nst) {
                const bool more = (st + 1) < nst;
                if (more) stage_load(st + 1);
#pragma unroll
                for (int cc = 0; cc < SC; ++cc) {
                    const int i = st * SC + cc;
                    const int u = (rr * SC + cc) % PF;
                    if (i < nck) {
                        compute(i, st & 1, cc, wreg[u], sreg[u], zreg[u]);
                        if (i + PF < nck) load_chunk(i + PF, wreg[u], sreg[u], zreg[u]);
                    }
                }
                if (more) stage_store((st + 1) & 1);
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
    if (a.ks == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = (ntb + j) * TILE_N + c;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + mt * 16 + g * 4 + r;
                    if (m < a.M && n < a.N) store_out(a, m, n, epilogue_value(a, acc[mt][j][r], n, rs[j]));
                }
            }
        return;
    }

    // split-K: store this split's float32 partial sums; the reduce kernel adds them
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int n = (ntb + j) * TILE_N + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + mt * 16 + g * 4 + r;
                if (m < a.M && n < a.Np) a.ws[(int64_t(kz) * a.M + m) * a.Np + n] = acc[mt][j][r];
            }
        }
}

}  // namespace ql
