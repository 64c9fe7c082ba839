// Large-tile kernel for prefill-sized M: activations AND packed weights are staged
// into an S-deep LDS ring by gfx950 direct buffer->LDS loads (buffer_load_dwordx4 ...
// lds), so nothing is staged through registers and several chunks are in flight.
//
// Workgroup = WM x WN wavefronts; a wavefront owns 16*MTW rows x 16*NTW columns, so a
// workgroup covers 16*MTW*WM rows and 16*NTW*WN columns.  One ring stage holds one chunk
// of the input dimension (128 inputs, 64 for INT8):
//   A  [k-step][8-wide slice][row] x 16 bytes: the A-fragment order, so each lane's
//      fragment is one conflict-free ds_read_b128;
//   B  the workgroup's packed 1 KiB weight tiles, copied verbatim (lane l's 16 bytes
//      land at l*16, exactly where the lane that decodes them reads).
// Per stage every wavefront waits for its own loads (s_waitcnt vmcnt), one barrier makes
// all of them visible and frees the oldest buffer, the loads of the stage S-1 ahead are
// issued, and the chunk is consumed: one ds_read_b128 per packed tile, register decode,
// MTW x NTW MFMAs per k-step.  Scales ride in registers (S-deep ring).  Out-of-range
// rows and inputs load as zero (ranged buffer loads).  Workgroups are numbered so that
// the ones sharing activation rows run on the same XCD (blocks are dealt round-robin to
// the 8 XCDs, each with its own L2).
#pragma once

#include <hip/hip_runtime.h>

#include "ql_common.hpp"
#include "ql_decode.hpp"

namespace ql {

// Workgroup barrier for the ring.  __syncthreads() carries a workgroup release fence,
// and with LDS written by buffer loads that fence waits for EVERY outstanding load of
// the wavefront (vmcnt(0)): the stages issued ahead would be drained at each chunk.
// Here each wavefront has already waited for exactly the loads the barrier publishes;
// its own LDS reads are waited for (lgkmcnt(0)) so the buffer the barrier frees is no
// longer being read, and the "memory" clobber keeps the compiler from moving LDS
// accesses or loads across it.
__device__ inline void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int FMT, bool ZP, int GS, int WM, int WN, int MTW, int NTW, int S>
__global__ void __launch_bounds__(64 * WM * WN) qgemm_lds_kernel(GemmArgs a) {
    constexpr int W = WM * WN;
    constexpr int CH = chunk_k(FMT);
    constexpr int STEPS = CH / 32;
    constexpr bool INTF = (FMT == FMT_INT4 || FMT == FMT_INT8);
    constexpr int SPC = INTF ? (GS <= STEPS ? STEPS / GS : 1) : 1;
    constexpr int MP = 16 * MTW * WM;               // rows of the workgroup tile
    constexpr int NTT = NTW * WN;                   // column tiles of the workgroup
    constexpr int A_BYTES = MP * CH * 2;
    constexpr int B_BYTES = NTT * TILE_BYTES;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int NA = A_BYTES / 1024;              // wave-wide A loads per stage
    constexpr int NB = NTT;                         // wave-wide B loads per stage
    static_assert(NA % W == 0 && NB % W == 0, "loads must split evenly over the wavefronts");
    constexpr int SL = INTF ? NTW * SPC * (ZP ? 2 : 1) : (FMT == FMT_MXFP4 ? NTW : 0);
    constexpr int PER_STAGE = NA / W + NB / W + SL;  // vector-memory ops per wavefront per stage
    static_assert(S >= 2 && S <= 4, "ring depth");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WN, wn = wv % WN;
    const int g = lane >> 4, c = lane & 15;

    // XCD-aware numbering: block b runs on XCD b % 8; give each XCD a contiguous range of
    // tiles, consecutive tiles sharing their row block
    const int total = gridDim.x;
    const int b = blockIdx.x;
    const int lin = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int nblocks = (a.ntiles + NTT - 1) / NTT;
    const int mtile = lin / nblocks, nblock = lin % nblocks;
    const int m0 = mtile * MP;
    const int nt0 = nblock * NTT;
    const int kz = blockIdx.y;
    const int kc0 = kz * a.cps;
    const int nck = min(a.kchunks - kc0, a.cps);

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, uint32_t(int64_t(a.M) * a.ldx * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, ZP ? a.z_bytes : 0u);
    const uint32_t s_shift = 16u * (c & 1);
    const uint32_t z_shift = 8u * ((c >> 1) & 3) + 4u * (c & 1);

    CbLut lut = {0u, 0u, 0u, 0u};
    if (FMT == FMT_CB4) lut = reinterpret_cast<const CbRecord *>(a.aux)->lut;

    f32x4 acc[MTW][NTW], tmp[MTW][NTW], xs[MTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        xs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            tmp[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    uint32_t sreg[S][NTW][SPC], zreg[S][NTW][SPC];

    // issue the loads of chunk i (relative) into ring buffer buf, scales into slot buf
    auto issue = [&](int i, int buf, uint32_t (&sq)[NTW][SPC], uint32_t (&zq)[NTW][SPC]) {
        const int kc = kc0 + i;
        uint8_t *base = lds + buf * STAGE;
        const int kbase = kc * CH;
#pragma unroll
        for (int q = 0; q < NA / W; ++q) {
            const int j = wv + W * q;                        // which 1 KiB of the A stage
            const int sidx = j * 64 + lane;                  // 16-byte slot = (block, row)
            const int row = sidx % MP, blk = sidx / MP;
            const int m = m0 + row, k = kbase + 32 * (blk >> 2) + 8 * (blk & 3);
            const uint32_t bad = (uint32_t(~(int32_t(k - a.K) >> 31)) | uint32_t(~(int32_t(m - a.M) >> 31))) &
                                 0x80000000u;
            const uint32_t off = ((uint32_t(m) * uint32_t(a.ldx) + uint32_t(k)) * 2u) | bad;
            ld128_lds(xr, off, base + j * 1024);
        }
#pragma unroll
        for (int q = 0; q < NB / W; ++q) {
            const int j = wv + W * q;
            const uint32_t tile = uint32_t(nt0 + j) * uint32_t(a.kchunks) + uint32_t(kc);
            ld128_lds(wr, tile * TILE_BYTES + lane * 16, base + A_BYTES + j * 1024);
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int ntg = nt0 + wn * NTW + j;
            if (FMT == FMT_MXFP4) {
                const uint32_t tile = uint32_t(ntg) * uint32_t(a.kchunks) + uint32_t(kc);
                sq[j][0] = ld32(sr, (tile * TILE_N + c) * 4);
            } else if (INTF) {
#pragma unroll
                for (int q = 0; q < SPC; ++q) {
                    const uint32_t grp = (GS <= STEPS) ? uint32_t(kc * (STEPS / GS) + q) : uint32_t(kc / (GS / STEPS));
                    const uint32_t rec = uint32_t(ntg) * uint32_t(a.ngroups) + grp;
                    sq[j][q] = ld32(sr, ((rec * TILE_N + c) * 2) & ~3u);
                    if (ZP) zq[j][q] = ld32(zr, (rec * 8 + (c >> 1)) & ~3u);
                }
            }
        }
    };

    const u32x4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 ones = as_bf16x8(ones_u);

    auto compute = [&](int i, int buf, const uint32_t (&sq)[NTW][SPC], const uint32_t (&zq)[NTW][SPC]) {
        const int kc = kc0 + i;
        const uint8_t *A = lds + buf * STAGE;
        const uint8_t *Bt = A + A_BYTES;
        u32x4 wq[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) wq[j] = *reinterpret_cast<const u32x4 *>(Bt + (wn * NTW + j) * 1024 + lane * 16);
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            bf16x8 af[MTW];
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
                af[mt] = *reinterpret_cast<const bf16x8 *>(A + ((t * 4 + g) * MP + (wm * MTW + mt) * 16 + c) * 16);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                u32x4 bw;
                if (FMT == FMT_INT4) bw = dec_int4(wq[j][t]);
                else if (FMT == FMT_INT8) bw = dec_int8(wq[j][2 * t], wq[j][2 * t + 1]);
                else if (FMT == FMT_MXFP4) bw = dec_mxfp4(wq[j][t], e8m0_to_f32((sq[j][0] >> (8 * t)) & 0xFFu));
                else bw = dec_cb4(wq[j][t], lut);
                const bf16x8 bv = as_bf16x8(bw);
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    if (INTF) tmp[mt][j] = mfma16x16x32(af[mt], bv, tmp[mt][j]);
                    else acc[mt][j] = mfma16x16x32(af[mt], bv, acc[mt][j]);
                }
            }
            if (INTF) {
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) xs[mt] = mfma16x16x32(af[mt], ones, xs[mt]);
                bool boundary;
                if (GS <= STEPS) boundary = ((t + 1) % GS) == 0;
                else boundary = (t == STEPS - 1) && (((kc + 1) % (GS / STEPS)) == 0);
                if (boundary) {
                    const int q = (GS <= STEPS) ? (t / GS) : 0;
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const uint32_t sbits = (sq[j][q] >> s_shift) & 0xFFFFu;
                        float s, off;
                        if (FMT == FMT_INT4) {
                            s = f16_bits_to_f32(sbits);
                            off = ZP ? 128.0f + float((zq[j][q] >> z_shift) & 0xFu) : 136.0f;
                        } else {
                            s = bf16_bits_to_f32(sbits);
                            off = 128.0f;
                        }
                        const float cz = -s * off;
#pragma unroll
                        for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                acc[mt][j][r] = fmaf(s, tmp[mt][j][r], acc[mt][j][r]);
                                acc[mt][j][r] = fmaf(cz, xs[mt][r], acc[mt][j][r]);
                            }
                            tmp[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
                    }
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) xs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };

    // ---- prologue: stages 0 .. S-2 in flight ----
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
        if (u < nck) issue(u, u, sreg[u], zreg[u]);

    // ---- main loop, unrolled by the ring depth so ring slots are compile-time ----
    for (int i0 = 0; i0 < nck; i0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int i = i0 + u;
            if (i < nck) {
                // loads issued after chunk i's: those of chunks i+1 .. min(i+S-2, nck-1)
                const int later = min(S - 2, nck - 1 - i);
                if (later >= 2) wait_vmcnt<2 * PER_STAGE>();
                else if (later == 1) wait_vmcnt<PER_STAGE>();
                else wait_vmcnt<0>();
                ring_barrier();
                if (i + S - 1 < nck) issue(i + S - 1, (u + S - 1) % S, sreg[(u + S - 1) % S], zreg[(u + S - 1) % S]);
                compute(i, u, sreg[u], zreg[u]);
            }
        }
    }

    // ---- epilogue ----
    float rs[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        rs[j] = 1.0f;
        if (FMT == FMT_CB4) {
            const int n = (nt0 + wn * NTW + j) * TILE_N + c;
            if (n < a.Np)
                rs[j] = reinterpret_cast<const float *>(a.s)[n] * reinterpret_cast<const CbRecord *>(a.aux)->inv_alpha;
        }
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int n = (nt0 + wn * NTW + j) * TILE_N + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + (wm * MTW + mt) * 16 + g * 4 + r;
                if (m >= a.M) continue;
                if (a.ks == 1) {
                    if (n >= a.N) continue;
                    float v = acc[mt][j][r];
                    if (FMT == FMT_CB4) v *= rs[j];
                    if (a.bias) v += bf16_bits_to_f32(a.bias[n]);
                    if (a.out_f32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
                    else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
                } else if (n < a.Np) {
                    a.ws[(int64_t(kz) * a.M + m) * a.Np + n] = acc[mt][j][r];
                }
            }
        }
}

}  // namespace ql
