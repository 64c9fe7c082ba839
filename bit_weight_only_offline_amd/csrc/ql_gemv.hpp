// Decode-shape kernel (M <= 16): split-K within the workgroup, wavefront-reduced.
//
// One workgroup owns NT column tiles (16*NT output columns) over the whole input
// dimension; its WK wavefronts split the chunks of the input dimension into WK
// contiguous runs (whole groups each).  Every wavefront streams its run through a
// private LDS ring, as many chunks ahead as the schedule's ring depth (two, or four for
// one column tile over a long input dimension), with direct buffer->LDS loads only: per chunk
// the packed weight tiles, the scale and zero-point words and the activation block
// (16 rows x one chunk of inputs; one load of rows, X1, when the batch fits it, which
// shrinks the stage so that more workgroups share a CU).  The activation loads read whole rows of the chunk
// (full 128-byte lines) and only the rows below M are requested; a XOR swizzle of the
// 16-byte pieces makes each A-fragment read a conflict-free ds_read_b128.  Nothing is
// loaded into registers, so every wait is explicit: a wavefront waits (vmcnt) only for
// the chunk it is about to use.  Weights are decoded in registers and accumulated with
// v_mfma_f32_16x16x32_bf16 (A rows at or beyond M never reach a stored output).  At the
// end the WK partial tiles are added in LDS in wavefront order -- a fixed order -- and
// the epilogue applies the codebook row scale and the bias and rounds to bf16.  No
// workspace, no cross-workgroup traffic.
//
// Fused SwiGLU input stage (SW, batches of at most SWIGLU_FUSE_MAX_M rows): the stage
// receives the up rows in the activation block and the gate rows in one more block, and
// the wavefront replaces each up value by h = bf16(up * silu(gate)) in LDS before it
// reads its A fragments -- the same arithmetic as the prologue kernel that materialises
// h for larger batches, so the two paths give the same linear.  Only the batch's rows
// are evaluated, 64 lanes across one chunk of them.  The stage then holds one activation
// load (its rows fit it), and the A fragments of rows past that load read its rows again
// (rows at or beyond M never reach a stored output).
//
// Codebook weights packed with the two-term operand (the record's split flag) issue a
// second MFMA per k-step on the residual operand, so the product carries about 16
// significant bits of each level instead of 8.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ql_common.hpp"
#include "ql_decode.hpp"

namespace ql {

template <int FMT, bool ZP, int GS, int NT, int WK, int PF, bool SW, bool X1>
__global__ void __launch_bounds__(64 * WK) qgemv_kernel(GemmArgs a) {
    constexpr int CH = chunk_k(FMT);
    constexpr int STEPS = CH / 32;
    constexpr bool INTF = (FMT == FMT_INT4 || FMT == FMT_INT8);
    constexpr int SPC = gemv_spc(FMT, GS);
    using XB = XBlock<FMT>;
    constexpr int NSS = gemv_scale_blocks(FMT, GS, NT);
    constexpr int NSZ = gemv_zero_blocks(FMT, ZP, GS, NT);
    constexpr int S_OFF = NT * TILE_BYTES;
    constexpr int Z_OFF = S_OFF + 256 * NSS;
    constexpr int X_OFF = Z_OFF + 256 * NSZ;
    constexpr int NI = (SW || X1) ? 1 : XB::NI;      // activation loads a stage holds
    constexpr int G_OFF = X_OFF + NI * 1024;          // gate rows (SW)
    constexpr int STAGE = gemv_stage_bytes(FMT, ZP, GS, NT, SW, X1);
    constexpr int S = gemv_ring_depth(FMT, ZP, GS, NT, WK, PF, SW, X1);
    static_assert(!(SW && X1), "one activation layout");
    static_assert(G_OFF + (SW ? 1024 : 0) == STAGE && S >= 1 && S <= 8, "stage layout");
    static_assert(gemv_rows_per_load(FMT) == XB::RPI, "rows per activation load");
    // fused SwiGLU: the batch's rows fit the first activation load; each lane forms HE
    // consecutive h values of one row
    constexpr int HE = SWIGLU_FUSE_MAX_M * CH / 64;
    static_assert(!SW || (SWIGLU_FUSE_MAX_M <= XB::RPI && (HE == 2 || HE == 4)), "fused SwiGLU rows");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];   // [WK][S][STAGE]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keep it scalar
    const int g = lane >> 4, c = lane & 15;
    const int ntb = blockIdx.x * NT;
    if (a.tile_map) {
        // grouped: blockIdx.y is a slot of up to 16 rows of one expert; those rows, their
        // output rows and the expert's packed buffers become this workgroup's problem
        const int slot = blockIdx.y;
        const int e = a.tile_map[2 * slot];
        if (e < 0) return;                               // unused slot: the whole workgroup
        const int row0 = a.offsets[e] + a.tile_map[2 * slot + 1];
        a.M = min(16, a.offsets[e + 1] - row0);
        a.x += int64_t(row0) * a.ldx;
        a.out = static_cast<uint8_t *>(a.out) + int64_t(row0) * a.N * (a.out_f32 ? 4 : 2);
        a.w += uint64_t(e) * a.w_stride;
        a.s += uint64_t(e) * a.s_stride;
        if (a.z) a.z += uint64_t(e) * a.z_stride;
        if (a.aux) a.aux += uint64_t(e) * CB_AUX_BYTES;
        if (a.bias) a.bias += int64_t(e) * a.N;
    }
    // this wavefront's run of chunks: cps per wavefront (a multiple of the group span)
    const int kc0 = wv * a.cps;
    const int nck = max(0, min(a.kchunks - kc0, a.cps));
    uint8_t *ring = lds + wv * (S * STAGE);

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, ZP ? a.z_bytes : 0u);
    // activations through a ranged buffer: rows >= M and inputs >= K read as zero
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint32_t(int64_t(a.M) * a.ldx * 2));
    const uint32_t s_shift = 16u * (c & 1);                       // this column's fp16/bf16 scale
    const uint32_t z_shift = 8u * ((c >> 1) & 3) + 4u * (c & 1);  // and its 4-bit zero-point

    CbLut lut = {0u, 0u, 0u, 0u}, lut2 = {0u, 0u, 0u, 0u};
    uint32_t split = 0;
    if (FMT == FMT_CB4) {
        const CbRecord *cr = reinterpret_cast<const CbRecord *>(a.aux);
        lut = cr->lut;
        lut2 = cr->lut_lo;
        split = uint32_t(__builtin_amdgcn_readfirstlane(int(cr->split)));
    }

    // ---- per-lane parts of the loads ----
    // activation loads actually issued: those holding a row below M (wave-uniform)
    const int nia = min(NI, (a.M + XB::RPI - 1) / XB::RPI);
    uint32_t xrow[NI];
    int xk[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int r = j * XB::RPI + lane / XB::P;
        const int pc = (lane % XB::P) ^ XB::xswz(r);
        xrow[j] = (r < a.M) ? uint32_t(r) * uint32_t(a.ldx) * 2u : 0x80000000u;   // bit 31: not fetched
        xk[j] = 8 * pc;
    }
    // this lane's A fragment of k-step t: row c, piece 4t + g
    uint32_t xfrag[STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t)
        xfrag[t] = uint32_t(X_OFF + XB::slot((SW || X1) ? c % XB::RPI : c, 4 * t + g));
    // scale / zero-point words: word e of a chunk's scale block is word (e % 8) of the
    // record of tile e / (8 SPC), group slot (e / 8) % SPC (MXFP4: column e % 16 of tile
    // e / 16); zero-point words likewise with 2 words per record
    int s_tile[NSS > 0 ? NSS : 1], s_q[NSS > 0 ? NSS : 1], s_w[NSS > 0 ? NSS : 1];
#pragma unroll
    for (int d = 0; d < NSS; ++d) {
        const int e = d * 64 + lane;
        if (FMT == FMT_MXFP4) {
            s_tile[d] = e / 16;
            s_q[d] = 0;
            s_w[d] = e % 16;
        } else {
            s_tile[d] = e / (8 * SPC);
            s_q[d] = (e / 8) % SPC;
            s_w[d] = e % 8;
        }
    }
    int z_tile[NSZ > 0 ? NSZ : 1], z_q[NSZ > 0 ? NSZ : 1], z_w[NSZ > 0 ? NSZ : 1];
#pragma unroll
    for (int d = 0; d < NSZ; ++d) {
        const int e = d * 64 + lane;
        z_tile[d] = e / (2 * SPC);
        z_q[d] = (e / 2) % SPC;
        z_w[d] = e % 2;
    }
    // the group record of group slot q in chunk kc
    auto group_of = [&](int kc, int q) -> uint32_t {
        return (GS <= STEPS) ? uint32_t(kc * (STEPS / GS) + q) : uint32_t(kc / (GS / STEPS));
    };

    // issue every load of chunk i (relative) into ring slot `slot`
    auto issue = [&](int i, int slot) {
        const int kc = kc0 + i;
        uint8_t *base = ring + slot * STAGE;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const uint32_t tile = uint32_t(ntb + j) * uint32_t(a.kchunks) + uint32_t(kc);
            ld128_lds(wr, tile * TILE_BYTES + lane * 16, base + j * TILE_BYTES);
        }
#pragma unroll
        for (int d = 0; d < NSS; ++d) {
            uint32_t off;
            if (FMT == FMT_MXFP4) {
                const uint32_t tile = uint32_t(ntb + s_tile[d]) * uint32_t(a.kchunks) + uint32_t(kc);
                off = (tile * TILE_N + uint32_t(s_w[d])) * 4;
            } else {
                const uint32_t rec = uint32_t(ntb + s_tile[d]) * uint32_t(a.ngroups) + group_of(kc, s_q[d]);
                off = rec * (TILE_N * 2) + uint32_t(s_w[d]) * 4;
            }
            if (s_tile[d] >= NT) off = 0x80000000u;                 // past this chunk's records
            ld32_lds(sr, off, base + S_OFF + d * 256);
        }
#pragma unroll
        for (int d = 0; d < NSZ; ++d) {
            const uint32_t rec = uint32_t(ntb + z_tile[d]) * uint32_t(a.ngroups) + group_of(kc, z_q[d]);
            uint32_t off = rec * 8 + uint32_t(z_w[d]) * 4;
            if (z_tile[d] >= NT) off = 0x80000000u;
            ld32_lds(zr, off, base + Z_OFF + d * 256);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            if (j < nia) {
                const int k = kc * CH + xk[j];
                const uint32_t past_k = uint32_t(~(int32_t(k - a.K) >> 31)) & 0x80000000u;   // k >= K
                ld128_lds(xr, (xrow[j] + uint32_t(k) * 2u) | past_k, base + X_OFF + j * 1024);
                // the gate half of the raw [up | gate] rows, same slots
                if (SW) ld128_lds(xr, (xrow[j] + uint32_t(a.K + k) * 2u) | past_k, base + G_OFF);
            }
        }
    };
    // vector-memory loads issued per chunk
    const int per_chunk = NT + NSS + NSZ + nia * (SW ? 2 : 1);
    // fused SwiGLU: this lane's HE values -- row hr, inputs hk .. hk+HE-1 of the chunk
    const int hr = (lane * HE) / CH, hk = (lane * HE) % CH;
    const uint32_t h_off = uint32_t(XB::slot(hr, hk / 8) + (hk % 8) * 2);

    f32x4 acc[NT], tmp[NT], xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        tmp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 ones = as_bf16x8(ones_u);

    auto compute = [&](int i, int slot, auto spl) {
        constexpr bool SPLIT = decltype(spl)::value;
        const int kc = kc0 + i;
        // chunk i has landed once only the chunks issued after it are outstanding
        wait_vmcnt_rt(per_chunk * min(S - 1, nck - 1 - i));
        compiler_fence();
        const uint8_t *base = ring + slot * STAGE;
        if constexpr (SW) {
            // h = bf16(up * silu(gate)) over the batch's rows of this chunk, in place of up
            // (LDS accesses of one wavefront complete in order: the fragment reads below
            // see these writes)
            uint8_t *hx = ring + slot * STAGE + X_OFF + h_off;
            const uint8_t *gx = ring + slot * STAGE + G_OFF + h_off;
            if constexpr (HE == 2) {
                *reinterpret_cast<uint32_t *>(hx) =
                    swiglu_pair(*reinterpret_cast<const uint32_t *>(hx), *reinterpret_cast<const uint32_t *>(gx));
            } else {
                const u32x2 up = *reinterpret_cast<const u32x2 *>(hx);
                const u32x2 gt = *reinterpret_cast<const u32x2 *>(gx);
                u32x2 h;
                h.x = swiglu_pair(up.x, gt.x);
                h.y = swiglu_pair(up.y, gt.y);
                *reinterpret_cast<u32x2 *>(hx) = h;
            }
        }
        u32x4 wq[NT];
        uint32_t sq[NT][SPC], zq[NT][SPC];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            wq[j] = *reinterpret_cast<const u32x4 *>(base + j * TILE_BYTES + lane * 16);
#pragma unroll
            for (int q = 0; q < SPC; ++q) {
                if (FMT == FMT_MXFP4) {
                    sq[j][q] = *reinterpret_cast<const uint32_t *>(base + S_OFF + (j * 16 + c) * 4);
                } else if (INTF) {
                    sq[j][q] = *reinterpret_cast<const uint32_t *>(base + S_OFF + ((j * SPC + q) * 8 + (c >> 1)) * 4);
                    if (ZP) zq[j][q] = *reinterpret_cast<const uint32_t *>(base + Z_OFF + ((j * SPC + q) * 2 + (c >> 3)) * 4);
                }
            }
        }
        // MXFP4: when no scale code of the chunk's words is 0 or 255 anywhere in the
        // wavefront (a wave-uniform test), each scale is its code shifted into the float32
        // exponent field, two instructions instead of six
        bool normal = false;
        if constexpr (FMT == FMT_MXFP4) {
            uint32_t sp = 0;
#pragma unroll
            for (int j = 0; j < NT; ++j) sp |= e8m0_special_bytes(sq[j][0]);
            normal = __builtin_amdgcn_ballot_w64(sp != 0) == 0;
        }
        auto ksteps = [&](auto normalc) {
        constexpr bool NORMAL = decltype(normalc)::value;
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const bf16x8 af = *reinterpret_cast<const bf16x8 *>(base + xfrag[t]);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                u32x4 bw;
                if (FMT == FMT_INT4) bw = dec_int4(wq[j][t]);
                else if (FMT == FMT_INT8) bw = dec_int8<false>(wq[j][2 * t], wq[j][2 * t + 1]);
                else if (FMT == FMT_MXFP4) {
                    const uint32_t e = (sq[j][0] >> (8 * t)) & 0xFFu;
                    bw = dec_mxfp4(wq[j][t], NORMAL ? e8m0_to_f32_normal(e) : e8m0_to_f32(e));
                } else {
                    bw = dec_cb4(wq[j][t], lut);
                    if constexpr (SPLIT) {
                        // the residual term first, then the leading term
                        acc[j] = mfma16x16x32(af, as_bf16x8(dec_cb4(wq[j][t], lut2)), acc[j]);
                    }
                }
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
                            off = 128.0f;                 // the operand here is bf16(u), u = q + 128
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
        if (FMT == FMT_MXFP4 && normal) ksteps(std::true_type{});
        else ksteps(std::false_type{});
    };

#pragma unroll
    for (int u = 0; u < S; ++u)
        if (u < nck) issue(u, u);
    auto main_loop = [&](auto spl) {
        for (int i0 = 0; i0 < nck; i0 += S) {
#pragma unroll
            for (int u = 0; u < S; ++u) {
                const int i = i0 + u;
                if (i < nck) {
                    compute(i, u, spl);
                    if (i + S < nck) {
                        // the slot is refilled: this wavefront's accesses of it must be complete
                        wait_lds();
                        issue(i + S, u);
                    }
                }
            }
        }
    };
    if (FMT == FMT_CB4 && split) main_loop(std::true_type{});
    else main_loop(std::false_type{});

    // ---- wavefront reduction in LDS (fixed order), then the epilogue ----
    __syncthreads();                      // every ring is drained: reuse the LDS
    float *red = reinterpret_cast<float *>(lds);   // [WK][NT][4][64]
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wv * NT + j) * 4 + r) * 64 + lane] = acc[j][r];
    __syncthreads();
    // output element e = (j, r, lane): row g*4 + r, column (ntb + j)*16 + c
    for (int e = tid; e < NT * 4 * 64; e += 64 * WK) {
        const int j = e / 256, r = (e / 64) % 4, l = e % 64;
        const int m = (l >> 4) * 4 + r, n = (ntb + j) * TILE_N + (l & 15);
        if (m >= a.M || n >= a.N) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WK; ++w) v += red[((w * NT + j) * 4 + r) * 64 + l];
        if (FMT == FMT_CB4) v *= reinterpret_cast<const float *>(a.s)[n] * reinterpret_cast<const CbRecord *>(a.aux)->inv_alpha;
        if (a.bias) v += bf16_bits_to_f32(a.bias[n]);
        if (a.out_f32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
        else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
    }
}

}  // namespace ql
