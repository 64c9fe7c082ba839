// Large-tile kernel for prefill-sized M: activations AND packed weights are staged
// into an S-deep LDS ring by gfx950 direct buffer->LDS loads (buffer_load_dwordx4 ...
// lds), so nothing is staged through registers and several chunks are in flight.
//
// Workgroup = WM x WN x WKK wavefronts; a wavefront owns 16*MTW rows x 16*NTW columns, so
// a workgroup covers 16*MTW*WM rows and 16*NTW*WN columns.  With WKK = 2 two wavefronts
// share each output tile and take alternate halves of every chunk's k-steps (two
// wavefronts per SIMD hide each other's LDS and decode latency); their accumulators are
// added in LDS, in a fixed order, before the epilogue.  One ring stage holds one chunk
// of the input dimension (128 inputs, 64 for INT8):
//   A  the tile's activation rows, loaded as whole row pieces of the chunk (full
//      128-byte lines per load) and XOR-swizzled so that each lane's fragment is one
//      conflict-free ds_read_b128 (XBlock);
//   B  the workgroup's packed 1 KiB weight tiles, copied verbatim (lane l's 16 bytes
//      land at l*16, exactly where the lane that decodes them reads).
// Per stage every wavefront waits for its own loads (s_waitcnt vmcnt), one barrier makes
// all of them visible and frees the oldest buffer, the loads of the stage S-1 ahead are
// issued, and the chunk is consumed: one read per packed tile (the lane's 16-byte record,
// or with two k-halves the 8 bytes of its half), register decode, MTW x NTW MFMAs per
// k-step.  Each wavefront's scale and zero-point words of the chunk
// ride in the same stage (4-byte direct loads), so every load of the loop goes to LDS
// and every wait is explicit.  Out-of-range
// rows and inputs load as zero (ranged buffer loads).  Workgroups are numbered so that
// the ones sharing activation rows run on the same XCD (blocks are dealt round-robin to
// the 8 XCDs, each with its own L2).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

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

template <int FMT, bool ZP, int GS, int WM, int WN, int WKK, int MTW, int NTW, int S>
__global__ void __launch_bounds__(64 * WM * WN * WKK) qgemm_lds_kernel(GemmArgs a) {
    constexpr int W = WM * WN * WKK;
    constexpr int CH = chunk_k(FMT);
    constexpr int STEPS = CH / 32;
    constexpr int SPW = STEPS / WKK;                // k-steps of a chunk per wavefront
    static_assert(SPW * WKK == STEPS, "k-steps split evenly");
    constexpr bool INTF = (FMT == FMT_INT4 || FMT == FMT_INT8);
    constexpr int SPC = INTF ? (GS <= STEPS ? STEPS / GS : 1) : 1;
    constexpr int MP = 16 * MTW * WM;               // rows of the workgroup tile
    constexpr int NTT = NTW * WN;                   // column tiles of the workgroup
    constexpr int A_BYTES = MP * CH * 2;
    constexpr int B_BYTES = NTT * TILE_BYTES;
    // every wavefront's scale / zero-point words of its NTW tiles (256-byte blocks)
    constexpr int NSS = gemv_scale_blocks(FMT, GS, NTW);
    constexpr int NSZ = gemv_zero_blocks(FMT, ZP, GS, NTW);
    constexpr int SCW = 256 * (NSS + NSZ);
    constexpr int STAGE = A_BYTES + B_BYTES + W * SCW;
    static_assert(STAGE == ring_stage_bytes(FMT, ZP, GS, WM, WN, WKK, MTW, NTW), "stage layout");
    constexpr int NA = A_BYTES / 1024;              // wave-wide A loads per stage
    constexpr int NB = NTT;                         // wave-wide B loads per stage
    static_assert(NA % W == 0, "activation loads split evenly over the wavefronts");

    static_assert(S >= 2 && S <= 6, "ring depth");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = WKK == 1 ? 0 : wv / (WM * WN);  // which k-steps of each chunk
    const int wm = (wv % (WM * WN)) / WN, wn = wv % WN;
    // B tiles are dealt round-robin, every wavefront issuing NBW loads: tile (wv + W q) mod
    // NB, so when W does not divide NB a few tiles are fetched twice (identical bytes to
    // the same LDS slot) and every wavefront waits for the same count
    constexpr int NBW = (NB + W - 1) / W;
    constexpr int PER_STAGE = NA / W + NBW + NSS + NSZ;   // vector-memory loads per wavefront per stage
    const int g = lane >> 4, c = lane & 15;

    // XCD-aware numbering: block b runs on XCD b % 8; give each XCD a contiguous range of
    // tiles, consecutive tiles sharing their row block
    const int total = gridDim.x;
    const int b = blockIdx.x;
    const int lin = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int nblocks = (a.ntiles + NTT - 1) / NTT;
    // few row blocks (small M): the row blocks of one column block are consecutive, so
    // they run on the same XCD and its L2 serves the weight tiles to all of them (the
    // activations are small and shared by every workgroup anyway); otherwise the column
    // blocks of one row block are consecutive and share the activation rows
    const int mtiles = a.tile_map ? a.slots : (a.M + MP - 1) / MP;
    const bool mfast = mtiles <= 4;
    const int mtile = mfast ? lin % mtiles : lin / nblocks;
    const int nblock = mfast ? lin / mtiles : lin % nblocks;
    int m0 = mtile * MP;
    if (a.tile_map) {
        // grouped: this slot's expert and row block; the expert's rows, output rows and
        // packed buffers become the whole problem of this workgroup
        const int e = a.tile_map[2 * mtile];
        if (e < 0) return;                               // unused slot: the whole workgroup
        m0 = a.tile_map[2 * mtile + 1];
        const int r0 = a.offsets[e];
        a.M = a.offsets[e + 1] - r0;
        a.x += int64_t(r0) * a.ldx;
        a.out = static_cast<uint8_t *>(a.out) + int64_t(r0) * a.N * (a.out_f32 ? 4 : 2);
        a.w += uint64_t(e) * a.w_stride;
        a.s += uint64_t(e) * a.s_stride;
        if (a.z) a.z += uint64_t(e) * a.z_stride;
        if (a.aux) a.aux += uint64_t(e) * CB_AUX_BYTES;
        if (a.bias) a.bias += int64_t(e) * a.N;
    }
    const int nt0 = nblock * NTT;
    const int kz = blockIdx.y;
    const int kc0 = kz * a.cps;
    const int nck = min(a.kchunks - kc0, a.cps);
    // Each workgroup walks its chunks starting at an offset set by its column block (a
    // multiple of the group span, wrapping around), so the workgroups that share a row
    // block of activations do not all miss on the same chunk at once.  The offset depends
    // on the column block only: a tile's summation order, hence its result, does not
    // depend on the grid it was launched in.
    constexpr int SPAN = (INTF && GS > STEPS) ? GS / STEPS : 1;
    const int rot = (nck > 0) ? int(((int64_t(nblock % 16) * nck) / 16) / SPAN) * SPAN : 0;
    auto chunk_of = [&](int i) { return kc0 + (i + rot < nck ? i + rot : i + rot - nck); };

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

    // per-lane parts of the ring loads that do not change from chunk to chunk: the
    // activation slot's row (rows >= M get bit 31: never fetched) and input offset, and
    // the weight tile's column block
    uint32_t a_off[NA / W];
    int a_k[NA / W];
#pragma unroll
    for (int q = 0; q < NA / W; ++q) {
        // load j covers rows j*RPI .. +RPI-1; this lane's row and (swizzled) piece
        using XB = XBlock<FMT>;
        const int row = (wv + W * q) * XB::RPI + lane / XB::P;
        const int m = m0 + row;
        a_k[q] = 8 * ((lane % XB::P) ^ XB::xswz(row));
        a_off[q] = (m < a.M) ? (uint32_t(m) * uint32_t(a.ldx) + uint32_t(a_k[q])) * 2u : 0x80000000u;
    }
    uint32_t b_off[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q)
        b_off[q] = uint32_t(nt0 + (wv + W * q) % NB) * uint32_t(a.kchunks) * TILE_BYTES + uint32_t(lane) * 16u;

    // scale / zero-point words: word e of this wavefront's scale block is word (e % 8) of
    // the record of its tile e / (8 SPC), group slot (e / 8) % SPC (MXFP4: column e % 16
    // of tile e / 16); zero-point words likewise with 2 words per record
    int s_tile[NSS > 0 ? NSS : 1], s_q[NSS > 0 ? NSS : 1], s_w[NSS > 0 ? NSS : 1];
#pragma unroll
    for (int d = 0; d < NSS; ++d) {
        const int e = d * 64 + lane;
        s_tile[d] = (FMT == FMT_MXFP4) ? e / 16 : e / (8 * SPC);
        s_q[d] = (FMT == FMT_MXFP4) ? 0 : (e / 8) % SPC;
        s_w[d] = (FMT == FMT_MXFP4) ? e % 16 : e % 8;
    }
    int z_tile[NSZ > 0 ? NSZ : 1], z_q[NSZ > 0 ? NSZ : 1], z_w[NSZ > 0 ? NSZ : 1];
#pragma unroll
    for (int d = 0; d < NSZ; ++d) {
        const int e = d * 64 + lane;
        z_tile[d] = e / (2 * SPC);
        z_q[d] = (e / 2) % SPC;
        z_w[d] = e % 2;
    }
    auto group_of = [&](int kc, int q) -> uint32_t {
        return (GS <= STEPS) ? uint32_t(kc * (STEPS / GS) + q) : uint32_t(kc / (GS / STEPS));
    };

    // only the last chunk can reach past K: this lane's pieces of it that do are marked
    // out of range once, here, and the mark is applied to that chunk alone.  The mark is
    // ORed into the finished offset: every in-range offset is below 2^31, and a
    // past-K offset added after the mark could carry out of bit 31 and wrap back into
    // the buffer when the activations fill nearly 2 GiB
    uint32_t tail_mask[NA / W];
#pragma unroll
    for (int q = 0; q < NA / W; ++q)
        tail_mask[q] = ((a.kchunks - 1) * CH + a_k[q] >= a.K) ? 0x80000000u : 0u;

    // issue the loads of chunk i (relative) into ring buffer buf
    auto issue = [&](int i, int buf) {
        const int kc = chunk_of(i);
        uint8_t *base = lds + buf * STAGE;
        const uint32_t kbase2 = uint32_t(kc * CH) * 2u;
        const uint32_t last = kc == a.kchunks - 1 ? 0xFFFFFFFFu : 0u;      // wave-uniform
#pragma unroll
        for (int q = 0; q < NA / W; ++q)
            ld128_lds(xr, (a_off[q] + kbase2) | (tail_mask[q] & last), base + (wv + W * q) * 1024);
#pragma unroll
        for (int q = 0; q < NBW; ++q)
            ld128_lds(wr, b_off[q] + uint32_t(kc) * TILE_BYTES, base + A_BYTES + ((wv + W * q) % NB) * 1024);
        uint8_t *sc = base + A_BYTES + B_BYTES + wv * SCW;
#pragma unroll
        for (int d = 0; d < NSS; ++d) {
            const uint32_t ntg = uint32_t(nt0 + wn * NTW + s_tile[d]);
            uint32_t off;
            if (FMT == FMT_MXFP4) off = ((ntg * uint32_t(a.kchunks) + uint32_t(kc)) * TILE_N + uint32_t(s_w[d])) * 4;
            else off = (ntg * uint32_t(a.ngroups) + group_of(kc, s_q[d])) * (TILE_N * 2) + uint32_t(s_w[d]) * 4;
            if (s_tile[d] >= NTW) off = 0x80000000u;               // past this wavefront's records
            ld32_lds(sr, off, sc + d * 256);
        }
#pragma unroll
        for (int d = 0; d < NSZ; ++d) {
            const uint32_t ntg = uint32_t(nt0 + wn * NTW + z_tile[d]);
            uint32_t off = (ntg * uint32_t(a.ngroups) + group_of(kc, z_q[d])) * 8 + uint32_t(z_w[d]) * 4;
            if (z_tile[d] >= NTW) off = 0x80000000u;
            ld32_lds(zr, off, sc + (NSS + d) * 256);
        }
    };

    const u32x4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 ones = as_bf16x8(ones_u);

    // this lane's A-fragment addresses inside a stage, for each of its k-steps of a chunk
    uint32_t a_frag[SPW][MTW];
#pragma unroll
    for (int tt = 0; tt < SPW; ++tt)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
            a_frag[tt][mt] = uint32_t(XBlock<FMT>::slot((wm * MTW + mt) * 16 + c, 4 * (kh * SPW + tt) + g));
    // this wavefront's words of a lane's 16-byte weight record: all four, or with two
    // k-halves the two of its half (4-bit formats: one word per k-step; INT8: two)
    constexpr int WPW = 4 / WKK;
    static_assert(WKK == 1 || WKK == 2, "one or two k-halves");

    auto compute = [&](int i, int buf) {
        const int kc = chunk_of(i);
        const uint8_t *A = lds + buf * STAGE;
        const uint8_t *Bt = A + A_BYTES;
        const uint8_t *sc = A + A_BYTES + B_BYTES + wv * SCW;
        uint32_t wq[NTW][WPW];
        uint32_t sq[NTW][SPC], zq[NTW][SPC];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const uint8_t *rec = Bt + (wn * NTW + j) * 1024 + lane * 16;
            if constexpr (WKK == 1) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(rec);
                wq[j][0] = v.x; wq[j][1] = v.y; wq[j][2] = v.z; wq[j][3] = v.w;
            } else {
                const u32x2 v = *reinterpret_cast<const u32x2 *>(rec + kh * 8);
                wq[j][0] = v.x; wq[j][1] = v.y;
            }
#pragma unroll
            for (int q = 0; q < SPC; ++q) {
                if (FMT == FMT_MXFP4) {
                    sq[j][q] = *reinterpret_cast<const uint32_t *>(sc + (j * 16 + c) * 4);
                } else if (INTF) {
                    sq[j][q] = *reinterpret_cast<const uint32_t *>(sc + ((j * SPC + q) * 8 + (c >> 1)) * 4);
                    if (ZP) zq[j][q] = *reinterpret_cast<const uint32_t *>(sc + NSS * 256 + ((j * SPC + q) * 2 + (c >> 3)) * 4);
                }
            }
        }
        // A fragments: with the codebook and MXFP4 (no group-sum registers) every k-step's
        // fragments of the chunk are read up front, so the reads of the later k-steps are
        // in flight during the MFMAs of the first; otherwise k-step by k-step
        constexpr int AHOLD = INTF ? 1 : SPW;
        bf16x8 afs[AHOLD][MTW];
        if constexpr (AHOLD > 1) {
#pragma unroll
            for (int tt = 0; tt < SPW; ++tt)
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) afs[tt][mt] = *reinterpret_cast<const bf16x8 *>(A + a_frag[tt][mt]);
            __builtin_amdgcn_sched_barrier(0);     // keep the reads ahead of the MFMAs
        }
#pragma unroll
        for (int tt = 0; tt < SPW; ++tt) {
            const int t = kh * SPW + tt;
            bf16x8 *af = afs[AHOLD > 1 ? tt : 0];
            if constexpr (AHOLD == 1) {
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) af[mt] = *reinterpret_cast<const bf16x8 *>(A + a_frag[tt][mt]);
            }
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                u32x4 bw;
                if (FMT == FMT_INT4) bw = dec_int4(wq[j][tt]);
                else if (FMT == FMT_INT8) bw = dec_int8<true>(wq[j][2 * tt], wq[j][2 * tt + 1]);
                else if (FMT == FMT_MXFP4) bw = dec_mxfp4(wq[j][tt], e8m0_to_f32((sq[j][0] >> (8 * t)) & 0xFFu));
                else bw = dec_cb4(wq[j][tt], lut);
                const bf16x8 bv = as_bf16x8(bw);
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    if (INTF) tmp[mt][j] = mfma16x16x32(af[mt], bv, tmp[mt][j]);
                    else acc[mt][j] = mfma16x16x32(af[mt], bv, acc[mt][j]);
                }
            }
            if (INTF) {
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt)
                    if (FMT == FMT_INT4) xs[mt] = mfma16x16x32(af[mt], ones, xs[mt]);   // INT8 codes are signed
                // fold the partial group sums at the last of this wavefront's steps in
                // the group (a group may span both halves of a chunk, or several chunks)
                bool boundary;
                if (GS <= STEPS) boundary = ((t + 1) % GS) == 0 || tt == SPW - 1;
                else boundary = (tt == SPW - 1) && (((kc + 1) % (GS / STEPS)) == 0);
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
                            off = 0.0f;                   // the operand is the signed code
                        }
                        const float cz = -s * off;
#pragma unroll
                        for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                acc[mt][j][r] = fmaf(s, tmp[mt][j][r], acc[mt][j][r]);
                                if (FMT == FMT_INT4) acc[mt][j][r] = fmaf(cz, xs[mt][r], acc[mt][j][r]);
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
        if (u < nck) issue(u, u);

    // ---- main loop, unrolled by the ring depth so ring slots are compile-time ----
    for (int i0 = 0; i0 < nck; i0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int i = i0 + u;
            if (i < nck) {
                // loads issued after chunk i's: those of chunks i+1 .. min(i+S-2, nck-1)
                const int later = min(S - 2, nck - 1 - i);
                if (later >= 4) wait_vmcnt<4 * PER_STAGE>();
                else if (later == 3) wait_vmcnt<3 * PER_STAGE>();
                else if (later == 2) wait_vmcnt<2 * PER_STAGE>();
                else if (later == 1) wait_vmcnt<PER_STAGE>();
                else wait_vmcnt<0>();
                ring_barrier();
                if (i + S - 1 < nck) issue(i + S - 1, (u + S - 1) % S);
                compute(i, u);
            }
        }
    }

    if constexpr (WKK > 1) {
        // add the k-halves in a fixed order: the wavefronts of the second half hand their
        // accumulators over through LDS (every ring is drained by now)
        static_assert(WM * WN * MTW * NTW * 1024 <= ring_lds_bytes(FMT, ZP, GS, WM, WN, WKK, MTW, NTW, S),
                      "hand-over fits the allocation");
        __syncthreads();
        float *red = reinterpret_cast<float *>(lds);
        const int slot = wv % (WM * WN);
        if (kh == 1) {
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[(((slot * MTW + mt) * NTW + j) * 4 + r) * 64 + lane] = acc[mt][j][r];
        }
        __syncthreads();
        if (kh != 0) return;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][j][r] += red[(((slot * MTW + mt) * NTW + j) * 4 + r) * 64 + lane];
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
    // a tile wholly inside the output, without a split: no per-element checks; the tile's
    // rows are one ranged buffer, each store = this lane's offset + a wave-uniform row
    // offset + a column-tile immediate, with the output type and the bias chosen once
    const int es = a.out_f32 ? 4 : 2;
    if (a.ks == 1 && m0 + MP <= a.M && (nt0 + NTT) * TILE_N <= a.N &&
        uint64_t(MP) * uint64_t(a.N) * uint64_t(es) < (uint64_t(1) << 32)) {
        float bj[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
            bj[j] = a.bias ? bf16_bits_to_f32(a.bias[(nt0 + wn * NTW + j) * TILE_N + c]) : 0.0f;
        auto emit = [&](auto f32c, auto biasc) {
            constexpr bool F32 = decltype(f32c)::value, BIAS = decltype(biasc)::value;
            constexpr uint32_t ES = F32 ? 4u : 2u;
            const __amdgpu_buffer_rsrc_t orc = make_uniform_rsrc(static_cast<uint8_t *>(a.out) + int64_t(m0) * a.N * ES,
                                                                 uint32_t(MP) * uint32_t(a.N) * ES);
            const uint32_t lane_off =
                (uint32_t(g * 4) * uint32_t(a.N) + uint32_t((nt0 + wn * NTW) * TILE_N + c)) * ES;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t row_off = uint32_t((wm * MTW + mt) * 16 + r) * uint32_t(a.N) * ES;
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        // the same expression as the checked path below
                        const float v = FMT == FMT_CB4 ? (BIAS ? fmaf(acc[mt][j][r], rs[j], bj[j]) : acc[mt][j][r] * rs[j])
                                                       : (BIAS ? acc[mt][j][r] + bj[j] : acc[mt][j][r]);
                        if (F32)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), orc, int(lane_off + j * TILE_N * ES),
                                                                  int(row_off), 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), orc,
                                                                  int(lane_off + j * TILE_N * ES), int(row_off), 0);
                    }
                }
        };
        if (a.out_f32) {
            if (a.bias) emit(std::true_type{}, std::true_type{});
            else emit(std::true_type{}, std::false_type{});
        } else {
            if (a.bias) emit(std::false_type{}, std::true_type{});
            else emit(std::false_type{}, std::false_type{});
        }
        return;
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
                    // codebook row scale and bias: one fused multiply-add when both apply
                    const float b = a.bias ? bf16_bits_to_f32(a.bias[n]) : 0.0f;
                    const float v = FMT == FMT_CB4 ? (a.bias ? fmaf(acc[mt][j][r], rs[j], b) : acc[mt][j][r] * rs[j])
                                                   : (a.bias ? acc[mt][j][r] + b : acc[mt][j][r]);
                    if (a.out_f32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
                    else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
                } else if (n < a.Np) {
                    a.ws[(int64_t(kz) * a.M + m) * a.Np + n] = acc[mt][j][r];
                }
            }
        }
}

}  // namespace ql
