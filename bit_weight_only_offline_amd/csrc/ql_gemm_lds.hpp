// Large-tile kernel for prefill-sized M: activations AND packed weights are staged
// into an S-deep LDS ring by gfx950 direct buffer->LDS loads (buffer_load_dwordx4 ...
// lds), so nothing is staged through registers and several chunks are in flight.
//
// Workgroup = WM x WN x WKK wavefronts; a wavefront owns 16*MTW rows x 16*NTW columns, so
// a workgroup covers 16*MTW*WM rows and 16*NTW*WN columns.  With WKK = 2 or 4, WKK
// wavefronts share each output tile and each takes its share of every chunk's k-steps
// (several wavefronts per SIMD hide each other's LDS and decode latency); their
// accumulators are added in LDS, in a fixed order, before the epilogue.  One ring stage holds one chunk
// of the input dimension (128 inputs, 64 for INT8):
//   A  the tile's activation rows, loaded as whole row pieces of the chunk (full
//      128-byte lines per load) and XOR-swizzled so that each lane's fragment is one
//      conflict-free ds_read_b128 (XBlock);
//   B  the workgroup's packed 1 KiB weight tiles, copied verbatim (lane l's 16 bytes
//      land at l*16, exactly where the lane that decodes them reads).
// Per stage every wavefront waits for its own loads (s_waitcnt vmcnt), one barrier makes
// all of them visible and frees a buffer, the loads of a stage further ahead are issued,
// and the chunk is consumed: one read per packed tile (the lane's 16-byte record, or
// with WKK k-parts the words of its part), register decode, MTW x NTW MFMAs per
// k-step.  INT4 / INT8 take the chunks one after the other; the codebook and MXFP4 are
// pipelined over k-steps (the next k-step's fragments are read during the current
// k-step's MFMAs, and the next chunk's barrier comes before the current chunk's last
// k-step).  Each wavefront's scale and zero-point words of the chunk
// ride in the same stage (4-byte direct loads), so every load of the loop goes to LDS
// and every wait is explicit.  Out-of-range
// rows and inputs load as zero (ranged buffer loads).  Workgroups are numbered so that
// the ones sharing activation rows run on the same XCD (blocks are dealt round-robin to
// the 8 XCDs, each with its own L2).  Codebook weights packed with the two-term operand
// (the record's split flag) issue a second MFMA per fragment on the residual operand.
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
// longer being read, and compiler fences keep LDS accesses and loads from moving across
// it.  The wait and the barrier are builtins, not assembly text: the compiler's own
// wait insertion then knows that every earlier LDS read has completed (after opaque
// assembly it waited again before the first use of each fragment read before the
// barrier, counting the reads issued after it).
__device__ inline void ring_barrier() {
    wait_lds();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

template <int FMT, bool ZP, int GS, int WM, int WN, int WKK, int MTW, int NTW, int S, bool CP>
__global__ void __launch_bounds__(64 * WM * WN * WKK) qgemm_lds_kernel(GemmArgs a) {
    constexpr int W = WM * WN * WKK;
    constexpr int CH = chunk_k(FMT);
    constexpr int STEPS = CH / 32;
    constexpr int SPW = STEPS / WKK;                // k-steps of a chunk per wavefront
    static_assert(SPW * WKK == STEPS, "k-steps split evenly");
    constexpr bool INTF = (FMT == FMT_INT4 || FMT == FMT_INT8);
    constexpr int SPC = INTF ? (GS <= STEPS ? STEPS / GS : 1) : 1;
    // k-steps of a chunk one wavefront multiplies, its record words per lane, and the
    // groups its k-steps fall in
    constexpr int SPWC = CP ? STEPS : SPW;
    constexpr int WPWC = CP ? 4 : 4 / WKK;
    constexpr int SPCW = INTF ? (GS <= SPWC ? SPWC / GS : 1) : 1;
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

    static_assert(S >= 2 && S <= 8, "ring depth");
    static_assert(!CP || WKK == 2, "chunk-parallel k-halves: two wavefronts per tile");
    constexpr int CS = CP ? 2 : 1;                  // chunks per ring stage
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = WKK == 1 ? 0 : wv / (WM * WN);  // which k-steps of each chunk
    const int wm = (wv % (WM * WN)) / WN, wn = wv % WN;
    // A loads and B tiles are dealt round-robin, every wavefront issuing NAW and NBW
    // loads: load (wv + W q) mod NA (NB), so when W does not divide NA (NB) a few are
    // fetched twice (identical bytes to the same LDS slot) and every wavefront waits for
    // the same count
    constexpr int NAW = (NA + W - 1) / W;
    constexpr int NBW = (NB + W - 1) / W;
    constexpr int PER_STAGE = NAW + NBW + NSS + NSZ;   // vector-memory loads per wavefront per stage
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

    const uint32_t x_bytes = uint32_t(int64_t(a.M) * a.ldx * 2);
    const uint32_t s_shift = 16u * (c & 1);
    const uint32_t z_shift = 8u * ((c >> 1) & 3) + 4u * (c & 1);

    CbLut lut = {0u, 0u, 0u, 0u}, lut2 = {0u, 0u, 0u, 0u};
    uint32_t split = 0;
    if (FMT == FMT_CB4) {
        const CbRecord *cr = reinterpret_cast<const CbRecord *>(a.aux);
        lut = cr->lut;
        lut2 = cr->lut_lo;
        split = uint32_t(__builtin_amdgcn_readfirstlane(int(cr->split)));
    }

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
    uint32_t a_off[NAW];
    int a_k[NAW];
#pragma unroll
    for (int q = 0; q < NAW; ++q) {
        // load j covers rows j*RPI .. +RPI-1; this lane's row and (swizzled) piece
        using XB = XBlock<FMT>;
        const int row = ((wv + W * q) % NA) * XB::RPI + lane / XB::P;
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
    // of tile e / 16); zero-point words likewise with 2 words per record.  The lane's
    // offsets for chunk 0 (a later chunk moves the descriptor's base); words past this
    // wavefront's records get bit 31: never fetched
    uint32_t s_off[NSS > 0 ? NSS : 1], z_off[NSZ > 0 ? NSZ : 1];
#pragma unroll
    for (int d = 0; d < NSS; ++d) {
        const int e = d * 64 + lane;
        const int tile = (FMT == FMT_MXFP4) ? e / 16 : e / (8 * SPC);
        const uint32_t ntg = uint32_t(nt0 + wn * NTW + tile);
        if (FMT == FMT_MXFP4) s_off[d] = (ntg * uint32_t(a.kchunks) * TILE_N + uint32_t(e % 16)) * 4;
        else s_off[d] = (ntg * uint32_t(a.ngroups) + uint32_t((e / 8) % SPC)) * (TILE_N * 2) + uint32_t(e % 8) * 4;
        if (tile >= NTW) s_off[d] = 0x80000000u;
    }
#pragma unroll
    for (int d = 0; d < NSZ; ++d) {
        const int e = d * 64 + lane;
        const int tile = e / (2 * SPC);
        z_off[d] = (uint32_t(nt0 + wn * NTW + tile) * uint32_t(a.ngroups) + uint32_t((e / 2) % SPC)) * 8 + uint32_t(e % 2) * 4;
        if (tile >= NTW) z_off[d] = 0x80000000u;
    }
    // first group of chunk kc (INT4 / INT8)
    auto group0 = [&](int kc) -> uint32_t {
        return (GS <= STEPS) ? uint32_t(kc * (STEPS / GS)) : uint32_t(kc / (GS / STEPS));
    };

    // only the last chunk can reach past K: this lane's pieces of it that do are marked
    // out of range once, here, and the mark is applied to that chunk alone.  The mark is
    // ORed into the finished offset: every in-range offset is below 2^31, and a
    // past-K offset added after the mark could carry out of bit 31 and wrap back into
    // the buffer when the activations fill nearly 2 GiB
    uint32_t tail_mask[NAW];
#pragma unroll
    for (int q = 0; q < NAW; ++q)
        tail_mask[q] = ((a.kchunks - 1) * CH + a_k[q] >= a.K) ? 0x80000000u : 0u;

    // issue the loads of chunk i (relative) into ring buffer buf.  The chunk's offsets go
    // into the descriptors' base addresses (scalar arithmetic), so the lanes' offsets stay
    // those of chunk 0 and a load takes no vector instruction
    auto issue = [&](int i, int buf) {
        const int kc = chunk_of(i);
        uint8_t *base = lds + buf * STAGE;
        const uint32_t xo = uint32_t(kc * CH) * 2u, wo = uint32_t(kc) * TILE_BYTES;
        const __amdgpu_buffer_rsrc_t xc = make_rsrc(a.x + kc * CH, x_bytes - xo);
        const __amdgpu_buffer_rsrc_t wc = make_rsrc(a.w + wo, a.w_bytes - wo);
        if (kc == a.kchunks - 1) {
#pragma unroll
            for (int q = 0; q < NAW; ++q)
                ld128_lds(xc, a_off[q] | tail_mask[q], base + ((wv + W * q) % NA) * 1024);
        } else {
#pragma unroll
            for (int q = 0; q < NAW; ++q) ld128_lds(xc, a_off[q], base + ((wv + W * q) % NA) * 1024);
        }
#pragma unroll
        for (int q = 0; q < NBW; ++q) ld128_lds(wc, b_off[q], base + A_BYTES + ((wv + W * q) % NB) * 1024);
        uint8_t *sc = base + A_BYTES + B_BYTES + wv * SCW;
        if constexpr (NSS > 0) {
            const uint32_t so = FMT == FMT_MXFP4 ? uint32_t(kc) * TILE_N * 4 : group0(kc) * (TILE_N * 2);
            const __amdgpu_buffer_rsrc_t sc_r = make_rsrc(a.s + so, a.s_bytes - so);
#pragma unroll
            for (int d = 0; d < NSS; ++d) ld32_lds(sc_r, s_off[d], sc + d * 256);
        }
        if constexpr (NSZ > 0) {
            const uint32_t zo = group0(kc) * 8;
            const __amdgpu_buffer_rsrc_t zc_r = make_rsrc(a.z + zo, a.z_bytes - zo);
#pragma unroll
            for (int d = 0; d < NSZ; ++d) ld32_lds(zc_r, z_off[d], sc + (NSS + d) * 256);
        }
    };

    const u32x4 ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8 ones = as_bf16x8(ones_u);

    // this lane's A-fragment address inside a stage for each of its k-steps of a chunk,
    // for the wavefront's first 16 rows: 16 rows further is one 16-row block further
    // (the swizzle repeats every 16 rows), a constant the reads add as an immediate
    using XB = XBlock<FMT>;
    static_assert(XB::slot(16 + 5, 3) == XB::slot(5, 3) + XB::BYTES, "16-row blocks are contiguous");
    uint32_t a_frag[SPWC];
#pragma unroll
    for (int tt = 0; tt < SPWC; ++tt)
        a_frag[tt] = uint32_t(XB::slot(wm * MTW * 16 + c, 4 * ((CP ? 0 : kh * SPW) + tt) + g));
    // this wavefront's words of a lane's 16-byte weight record (WPWC): all four, or with
    // WKK k-parts splitting each chunk the 4 / WKK of its part (4-bit formats: one word
    // per k-step; INT8: two)
    static_assert(WKK == 1 || WKK == 2 || WKK == 4, "one, two or four k-parts");

    // ring steps: one chunk each, or with CP two (chunks 2r and 2r+1 of ring step r in
    // chunk slots 2v and 2v+1 of ring slot v = r % S, one per k-half)
    const int nrs = CP ? (nck + 1) / 2 : nck;
    // chunks in ring steps a0 .. b0 (none when b0 < a0)
    auto chunks_in = [&](int a0, int b0) {
        return b0 < a0 ? 0 : CP ? min(2 * (b0 + 1), nck) - 2 * a0 : b0 - a0 + 1;
    };
    auto cslot = [&](int v) { return CP ? 2 * v + kh : v; };    // this wavefront's chunk slot
    auto issue_rs = [&](int r, int v) {
        if constexpr (CP) {
            issue(2 * r, 2 * v);
            if (2 * r + 1 < nck) issue(2 * r + 1, 2 * v + 1);
        } else {
            issue(r, v);
        }
    };

    // INT4 / INT8: one chunk, k-step by k-step; each group's partial sums collect in
    // tmp and are folded into acc with the group's scale (and offset) at the group's end
    auto compute = [&](int i, int buf) {
        const int kc = chunk_of(i);
        const uint8_t *A = lds + buf * STAGE;
        const uint8_t *Bt = A + A_BYTES;
        const uint8_t *sc = A + A_BYTES + B_BYTES + wv * SCW;
        uint32_t wq[NTW][WPWC];
        // scale words of the groups this wavefront's k-steps fall in, indexed by the
        // step's local group (a compile-time index: a run-time one would put the array
        // in scratch memory)
        uint32_t sq[NTW][SPCW], zq[NTW][SPCW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const uint8_t *rec = Bt + (wn * NTW + j) * 1024 + lane * 16;
            if constexpr (WPWC == 4) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(rec);
                wq[j][0] = v.x; wq[j][1] = v.y; wq[j][2] = v.z; wq[j][3] = v.w;
            } else if constexpr (WPWC == 2) {
                const u32x2 v = *reinterpret_cast<const u32x2 *>(rec + kh * 8);
                wq[j][0] = v.x; wq[j][1] = v.y;
            } else {
                wq[j][0] = *reinterpret_cast<const uint32_t *>(rec + kh * 4);
            }
#pragma unroll
            for (int q = 0; q < SPCW; ++q) {
                // the chunk's group slot: this wavefront's q-th group, or the one group
                // its steps lie in
                const int kq = CP ? 0 : kh * SPW;          // first k-step of this wavefront
                const int qg = GS > STEPS ? 0 : GS <= SPWC ? kq / GS + q : kq / GS;
                sq[j][q] = *reinterpret_cast<const uint32_t *>(sc + ((j * SPC + qg) * 8 + (c >> 1)) * 4);
                if (ZP) zq[j][q] = *reinterpret_cast<const uint32_t *>(sc + NSS * 256 + ((j * SPC + qg) * 2 + (c >> 3)) * 4);
            }
        }
#pragma unroll
        for (int tt = 0; tt < SPWC; ++tt) {
            bf16x8 af[MTW];
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) af[mt] = *reinterpret_cast<const bf16x8 *>(A + a_frag[tt] + mt * XB::BYTES);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const bf16x8 bv = as_bf16x8(FMT == FMT_INT4 ? dec_int4(wq[j][tt])
                                                            : dec_int8<true>(wq[j][2 * tt], wq[j][2 * tt + 1]));
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) tmp[mt][j] = mfma16x16x32(af[mt], bv, tmp[mt][j]);
            }
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
                if (FMT == FMT_INT4) xs[mt] = mfma16x16x32(af[mt], ones, xs[mt]);   // INT8 codes are signed
            // fold the partial group sums at the last of this wavefront's steps in the
            // group (a group may span both halves of a chunk, or several chunks; with CP
            // a wavefront sees every other chunk of a group, the last of them at chunk
            // span-2 or span-1 of the group)
            bool boundary;
            if (GS <= SPWC) boundary = ((tt + 1) % GS) == 0;
            else if (GS <= STEPS) boundary = tt == SPWC - 1;
            else if (CP) boundary = (tt == SPWC - 1) && ((kc % (GS / STEPS)) >= GS / STEPS - 2);
            else boundary = (tt == SPWC - 1) && (((kc + 1) % (GS / STEPS)) == 0);
            if (boundary) {
                const int q = GS <= SPWC ? tt / GS : 0;
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
    };

    // wait until chunk i's loads (this wavefront's) have landed, given how many chunks'
    // loads were issued after them (at most 6 counted).  Away from the end of the input
    // dimension that is every later ring step in flight, CS (S - 2) chunks: tested first,
    // so the steady state takes one compare instead of the whole ladder
    constexpr int STEADY = CS * (S - 2) < 6 ? CS * (S - 2) : 6;
    auto wait_later = [&](int later) {
        if (later >= STEADY) wait_vmcnt<STEADY * PER_STAGE>();
        else if (later >= 6) wait_vmcnt<6 * PER_STAGE>();
        else if (later == 5) wait_vmcnt<5 * PER_STAGE>();
        else if (later == 4) wait_vmcnt<4 * PER_STAGE>();
        else if (later == 3) wait_vmcnt<3 * PER_STAGE>();
        else if (later == 2) wait_vmcnt<2 * PER_STAGE>();
        else if (later == 1) wait_vmcnt<PER_STAGE>();
        else wait_vmcnt<0>();
    };
    if constexpr (INTF) {
        // ---- prologue: ring steps 0 .. S-2 in flight ----
#pragma unroll
        for (int u = 0; u < S - 1; ++u)
            if (u < nrs) issue_rs(u, u);

        // ---- main loop, unrolled by the ring depth so ring slots are compile-time ----
        for (int r0 = 0; r0 < nrs; r0 += S) {
#pragma unroll
            for (int u = 0; u < S; ++u) {
                const int r = r0 + u;
                if (r < nrs) {
                    // loads issued after step r's: those of steps r+1 .. min(r+S-2, nrs-1)
                    wait_later(chunks_in(r + 1, min(r + S - 2, nrs - 1)));
                    ring_barrier();
                    if (r + S - 1 < nrs) issue_rs(r + S - 1, (u + S - 1) % S);
                    if (!CP) compute(r, u);
                    else if (2 * r + kh < nck) compute(2 * r + kh, cslot(u));
                }
            }
        }
    } else {
        // Codebook and MXFP4: pipelined over k-steps.  The A fragments of the next k-step
        // are read during the MFMAs of the current one.  The ring barrier of step r+1
        // comes before the last k-step of step r: by then every wavefront holds the rest
        // of step r in registers, so its ring slot is refilled (with step r+S) at that
        // barrier, and step r+1's weight words and first A fragments are read while the
        // last MFMAs of step r run.
        // fragment double buffer by k-step parity; with one k-step per wavefront the next
        // step's fragments go to the other buffer and are moved over after the step
        static_assert(SPWC == 1 || SPWC % 2 == 0, "fragment double buffer by k-step parity");
        constexpr int CL = (SPWC - 1) & 1;      // buffer of a ring step's last k-step
        constexpr int NX = SPWC == 1 ? 1 : 0;   // buffer the next ring step's first fragments go to
        uint32_t wq[NTW][WPWC], wqn[NTW][WPWC], sw[NTW], swn[NTW];
        bf16x8 af[2][MTW];
        auto read_b = [&](int slot, uint32_t (&w)[NTW][WPWC], uint32_t (&sx)[NTW]) {
            const uint8_t *Bt = lds + slot * STAGE + A_BYTES;
            const uint8_t *sc = Bt + B_BYTES + wv * SCW;
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const uint8_t *rec = Bt + (wn * NTW + j) * 1024 + lane * 16;
                if constexpr (WPWC == 4) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(rec);
                    w[j][0] = v.x; w[j][1] = v.y; w[j][2] = v.z; w[j][3] = v.w;
                } else if constexpr (WPWC == 2) {
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(rec + kh * 8);
                    w[j][0] = v.x; w[j][1] = v.y;
                } else {
                    w[j][0] = *reinterpret_cast<const uint32_t *>(rec + kh * 4);
                }
                sx[j] = FMT == FMT_MXFP4 ? *reinterpret_cast<const uint32_t *>(sc + (j * 16 + c) * 4) : 0u;
            }
        };
        auto read_a = [&](int slot, int tt, bf16x8 (&f)[MTW]) {
            const uint8_t *A = lds + slot * STAGE;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) f[mt] = *reinterpret_cast<const bf16x8 *>(A + a_frag[tt] + mt * XB::BYTES);
        };
        // one k-step's MFMAs, with the register decode of each weight fragment
        // interleaved: the first fragment's decode, then each MFMA followed by up to two
        // VALU instructions and one of the NRD fragment reads issued before it (left to
        // itself the scheduler emits the MFMAs in bursts and the VALU work between them)
        auto step = [&](const bf16x8 (&f)[MTW], const uint32_t (&w)[NTW][WPWC], const uint32_t (&sx)[NTW], int tt,
                        auto spl, auto nrdc) {
            constexpr bool SPLIT = decltype(spl)::value;
            constexpr int NRD = decltype(nrdc)::value;
            const int t = (CP ? 0 : kh * SPW) + tt;    // the k-step within the chunk
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                u32x4 bw;
                if (FMT == FMT_MXFP4) bw = dec_mxfp4(w[j][tt], e8m0_to_f32((sx[j] >> (8 * t)) & 0xFFu));
                else {
                    bw = dec_cb4(w[j][tt], lut);
                    if constexpr (SPLIT) {
                        // the residual term first, then the leading term
                        const bf16x8 bl = as_bf16x8(dec_cb4(w[j][tt], lut2));
#pragma unroll
                        for (int mt = 0; mt < MTW; ++mt) acc[mt][j] = mfma16x16x32(f[mt], bl, acc[mt][j]);
                    }
                }
                const bf16x8 bv = as_bf16x8(bw);
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) acc[mt][j] = mfma16x16x32(f[mt], bv, acc[mt][j]);
            }
            constexpr int NMF = NTW * MTW * (SPLIT ? 2 : 1);
            __builtin_amdgcn_sched_group_barrier(0x002, FMT == FMT_MXFP4 ? 8 : (SPLIT ? 28 : 14), 0);
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        };
        using Mid = std::integral_constant<int, MTW>;
        using Last = std::integral_constant<int, MTW + NTW * (FMT == FMT_MXFP4 ? 2 : 1)>;

        // ---- prologue: ring steps 0 .. S-2 in flight; step 0's words and first fragments ----
#pragma unroll
        for (int u = 0; u < S - 1; ++u)
            if (u < nrs) issue_rs(u, u);
        wait_later(chunks_in(1, min(S - 2, nrs - 1)));
        ring_barrier();
        if (S - 1 < nrs) issue_rs(S - 1, S - 1);
        read_b(cslot(0), wq, sw);
        read_a(cslot(0), 0, af[0]);

        // ---- main loop, unrolled by the ring depth so ring slots are compile-time ----
        auto main_loop = [&](auto spl) {
            for (int r0 = 0; r0 < nrs; r0 += S) {
#pragma unroll
                for (int u = 0; u < S; ++u) {
                    const int r = r0 + u;
                    if (r < nrs) {
                        // with CP and an odd chunk count the last step has no chunk for
                        // the second k-half (wave-uniform)
                        const bool act = !CP || 2 * r + kh < nck;
#pragma unroll
                        for (int tt = 0; tt < SPWC - 1; ++tt) {
                            read_a(cslot(u), tt + 1, af[(tt + 1) & 1]);
                            if (act) step(af[tt & 1], wq, sw, tt, spl, Mid{});
                        }
                        // step r+1: loads issued after its own are those of steps
                        // r+2 .. min(r+S-1, nrs-1); past the last step the reads below
                        // fetch a stale slot, unused
                        wait_later(chunks_in(r + 2, min(r + S - 1, nrs - 1)));
                        ring_barrier();
                        if (r + S < nrs) issue_rs(r + S, u);
                        read_b(cslot((u + 1) % S), wqn, swn);
                        read_a(cslot((u + 1) % S), 0, af[NX]);
                        if (act) step(af[CL], wq, sw, SPWC - 1, spl, Last{});
                        if constexpr (SPWC == 1) {
#pragma unroll
                            for (int mt = 0; mt < MTW; ++mt) af[0][mt] = af[1][mt];
                        }
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            sw[j] = swn[j];
#pragma unroll
                            for (int q = 0; q < WPWC; ++q) wq[j][q] = wqn[j][q];
                        }
                    }
                }
            }
        };
        if (FMT == FMT_CB4 && split) main_loop(std::true_type{});
        else main_loop(std::false_type{});
    }

    if constexpr (WKK > 1) {
        // add the k-parts in a fixed order, ((part 0 + part 1) + part 2) + part 3: the
        // wavefronts of the later parts hand their accumulators over through LDS (every
        // ring is drained by now)
        constexpr int HB = WM * WN * MTW * NTW * 256;   // floats of one part's hand-over
        static_assert((WKK - 1) * HB * 4 <= ring_lds_bytes(FMT, ZP, GS, WM, WN, WKK, MTW, NTW, S, CS),
                      "hand-over fits the allocation");
        __syncthreads();
        float *red = reinterpret_cast<float *>(lds);
        const int slot = wv % (WM * WN);
        if (kh != 0) {
            float *dst = red + (kh - 1) * HB;
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(((slot * MTW + mt) * NTW + j) * 4 + r) * 64 + lane] = acc[mt][j][r];
        }
        __syncthreads();
        if (kh != 0) return;
#pragma unroll
        for (int p = 0; p < WKK - 1; ++p)
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[mt][j][r] += red[p * HB + (((slot * MTW + mt) * NTW + j) * 4 + r) * 64 + lane];
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
    // split-K partials: raw sums into the workspace (the reduction applies scale and bias)
    if (a.ks != 1) {
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int n = (nt0 + wn * NTW + j) * TILE_N + c;
                if (n >= a.Np) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + (wm * MTW + mt) * 16 + g * 4 + r;
                    if (m < a.M) a.ws[(int64_t(kz) * a.M + m) * a.Np + n] = acc[mt][j][r];
                }
            }
        return;
    }
    // an edge tile: per-element bounds, with the output type and the bias chosen once so
    // that each unrolled element is one check and one store (a body small enough for the
    // loops to unroll fully at every tile shape, which keeps acc in registers)
    auto emit_edge = [&](auto f32c, auto biasc) {
        constexpr bool F32 = decltype(f32c)::value, BIAS = decltype(biasc)::value;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int n = (nt0 + wn * NTW + j) * TILE_N + c;
                if (n >= a.N) continue;
                // codebook row scale and bias: one fused multiply-add when both apply
                const float b = BIAS ? bf16_bits_to_f32(a.bias[n]) : 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + (wm * MTW + mt) * 16 + g * 4 + r;
                    if (m >= a.M) continue;
                    const float v = FMT == FMT_CB4 ? (BIAS ? fmaf(acc[mt][j][r], rs[j], b) : acc[mt][j][r] * rs[j])
                                                   : (BIAS ? acc[mt][j][r] + b : acc[mt][j][r]);
                    if (F32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
                    else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
                }
            }
    };
    if (a.out_f32) {
        if (a.bias) emit_edge(std::true_type{}, std::true_type{});
        else emit_edge(std::true_type{}, std::false_type{});
    } else {
        if (a.bias) emit_edge(std::false_type{}, std::true_type{});
        else emit_edge(std::false_type{}, std::false_type{});
    }
}

}  // namespace ql
