// INT8-compute linear (W4A8 / W8A8): the activation rows are quantised to INT8 on the fly,
// one float32 scale per row, and the products run on the INT8 matrix cores
// (v_mfma_i32_16x16x64_i8) with exact int32 sums per weight group; the group scales and
// the row scale are applied in float32.  (AutoRound Kernel package description,
// "1. Linear": "Key Features", W4A8 / W2A8 rescale in the style of QQQ: low-bit weights
// re-scaled to INT8 and computed by an INT8 GEMM instead of dequantising to 16 bits;
// "Supported Data Types": INT8 compute includes dynamic activation quantisation and the
// results are dequantised to floating point.)
//
// Weights are the symmetric INT4 or INT8 packed layout of qlinear_pack() unchanged.  A
// lane's 16-byte B operand of one 64-input step is taken straight from its packed
// record: INT4 nibbles (offset-binary u = q + 8) become signed bytes by
// ((u + 0x78) ^ 0x80) after a mask and a shift, INT8 offset-binary bytes by ^ 0x80.
// The order of the values inside the operand follows the record (INT4: 0,4,1,5,2,6,3,7
// of each 8-input run, from the nibble order of the record word); the quantised
// activation rows are written in exactly that order, so A and B agree element by
// element and the matrix core sums the right products.
//
// Quantised activation row layout (one row per token, Kp bytes, Kp = K padded to the
// weight chunk, zero past K): input k = 64 b + 32 t + 8 g + j goes to byte
// 64 b + 16 g + 8 t + e(j), with e(j) = j for INT8 weights and 2 (j mod 4) + j / 4 for
// INT4 weights.  Lane (g, c) of a 64-input step then reads one 16-byte piece.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "ql_common.hpp"
#include "ql_decode.hpp"
#include "ql_gemm_lds.hpp"
#include "ql_launch.hpp"

namespace ql {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// byte position of input k inside a quantised activation row
__host__ __device__ constexpr int a8_pos(int k, int layout) {
    // layout 0: natural order; 1: for INT4 weights; 2: for INT8 weights
    return layout == 0 ? k
                       : ((k & ~63) | (((k >> 3) & 3) << 4) | (((k >> 5) & 1) << 3) |
                          (layout == 1 ? ((k & 3) * 2 + ((k >> 2) & 1)) : (k & 7)));
}

// One workgroup (256 threads) per row: amax over the row (bf16 magnitudes compared as
// integers, a lane-shuffle then a cross-wave reduction), the row scale s = amax / 127,
// then codes clamp(rint(x / s), -127, 127) in float32.  Threads own 8 consecutive inputs
// per 16-byte load, B loads in flight per batch of 2048 B inputs; rows of up to 2048 B
// inputs stay in registers between the two passes.  Rows are written Kp bytes long
// (zeros past K).
template <int LAYOUT>
__global__ void __launch_bounds__(256) quant_act_kernel(const uint16_t *__restrict__ x, int M, int K, int Kp,
                                                        int8_t *__restrict__ codes, float *__restrict__ scales) {
    constexpr int B = 4;                                  // loads per thread per batch
    constexpr int SPAN = 256 * 8;                         // inputs per load round
    __shared__ uint32_t red[4];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int m = blockIdx.x;
    const uint16_t *row = x + int64_t(m) * K;
    const bool resident = Kp <= SPAN * B;
    u32x4 v[B];
    uint32_t am = 0;
    for (int b0 = 0; b0 < K; b0 += SPAN * B) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int k8 = b0 + SPAN * i + 8 * t;
            v[i] = k8 < K ? *reinterpret_cast<const u32x4 *>(row + k8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < B; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) am = max(am, max(v[i][w] & 0x7FFFu, (v[i][w] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) am = max(am, uint32_t(__shfl_xor(int(am), d, 64)));
    if (lane == 0) red[wv] = am;
    __syncthreads();
    am = max(max(red[0], red[1]), max(red[2], red[3]));
    const float s = __fdiv_rn(bf16_bits_to_f32(am), 127.0f);
    if (t == 0) scales[m] = s;
    int8_t *out = codes + int64_t(m) * Kp;
    for (int b0 = 0; b0 < Kp; b0 += SPAN * B) {
        if (!resident) {
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const int k8 = b0 + SPAN * i + 8 * t;
                v[i] = k8 < K ? *reinterpret_cast<const u32x4 *>(row + k8) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int k8 = b0 + SPAN * i + 8 * t;
            if (k8 >= Kp) break;
            uint32_t q8[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xv = bf16_bits_to_f32((v[i][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
                const float q = s > 0.0f ? fminf(fmaxf(rintf(__fdiv_rn(xv, s)), -127.0f), 127.0f) : 0.0f;
                const int e = a8_pos(j, LAYOUT);          // position inside the 8-byte run
                q8[e >> 2] |= (uint32_t(int(q)) & 0xFFu) << (8 * (e & 3));
            }
            *reinterpret_cast<u32x2 *>(out + a8_pos(k8, LAYOUT)) = u32x2{q8[0], q8[1]};
        }
    }
}

struct A8Args {
    const int8_t *xq;        // quantised activations [M, Kp]
    const float *xs;         // row scales [M]
    const uint8_t *w, *s;    // packed weight and scales
    const uint16_t *bias;    // bf16 [N] or null
    void *out;               // [M, N] bf16 or float32
    int M, N, Kp, kchunks, ngroups, ntiles, out_f32;
    uint32_t w_bytes, s_bytes;
};

// 16 signed bytes of one 64-input step from a lane's packed record
template <int WF>
__device__ inline i32x4 b_operand(const u32x4 &rec, int step) {
    if (WF == FMT_INT4) {
        const uint32_t w0 = rec[2 * step], w1 = rec[2 * step + 1];
        const uint32_t m = 0x0F0F0F0Fu, bias = 0x78787878u, flip = 0x80808080u;
        i32x4 r;
        r.x = int32_t(((w0 & m) + bias) ^ flip);
        r.y = int32_t((((w0 >> 4) & m) + bias) ^ flip);
        r.z = int32_t(((w1 & m) + bias) ^ flip);
        r.w = int32_t((((w1 >> 4) & m) + bias) ^ flip);
        return r;
    } else {
        const uint32_t flip = 0x80808080u;
        return i32x4{int32_t(rec.x ^ flip), int32_t(rec.y ^ flip), int32_t(rec.z ^ flip), int32_t(rec.w ^ flip)};
    }
}

// Ring kernel on the INT8 matrix cores: WM x WN wavefronts, each 16*MTW rows x 16*NTW
// columns; one ring stage = one weight chunk (128 inputs for INT4, 64 for INT8) of the
// quantised activation rows (XOR-swizzled 16-byte pieces, full-line loads), the packed
// tiles and each wavefront's scale words, all by direct buffer->LDS loads.  GS is the
// group in 32-input steps (2, 4 or 8).
template <int WF, int GS, int WM, int WN, int MTW, int NTW, int S>
__global__ void __launch_bounds__(64 * WM * WN) qgemm_a8_kernel(A8Args a) {
    constexpr int W = WM * WN;
    constexpr int CH = chunk_k(WF);
    constexpr int STEPS = CH / 32;                  // 32-input steps (scale bookkeeping)
    constexpr int ST8 = CH / 64;                    // 64-input matrix-core steps
    constexpr int SPC = GS <= STEPS ? STEPS / GS : 1;
    static_assert(GS >= 2, "groups of at least 64 inputs");
    constexpr int P = CH / 16;                      // 16-byte pieces of a row's chunk
    constexpr int RPI = 64 / P;                     // rows per 1 KiB load
    constexpr int MP = 16 * MTW * WM;
    constexpr int NTT = NTW * WN;
    constexpr int A_BYTES = MP * CH;
    constexpr int B_BYTES = NTT * TILE_BYTES;
    constexpr int NSS = gemv_scale_blocks(WF, GS, NTW);
    constexpr int SCW = 256 * NSS;
    constexpr int STAGE = A_BYTES + B_BYTES + W * SCW;
    constexpr int NA = A_BYTES / 1024;
    constexpr int NB = NTT;
    constexpr int NBW = (NB + W - 1) / W;
    // loads are dealt round-robin, every wavefront issuing NAW (NBW) of them: load
    // (wv + W q) mod NA, so when W does not divide NA a few are issued twice (identical
    // bytes to the same LDS slot) and every wavefront waits for the same count
    constexpr int NAW = (NA + W - 1) / W;
    constexpr int PER_STAGE = NAW + NBW + NSS;
    static_assert(S >= 2 && S <= 6, "ring depth");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WN, wn = wv % WN;
    const int g = lane >> 4, c = lane & 15;

    // XCD-aware numbering (block b runs on XCD b % 8), as in the bf16 ring kernel
    const int total = gridDim.x, b = blockIdx.x;
    const int lin = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int nblocks = (a.ntiles + NTT - 1) / NTT;
    const int mtiles = (a.M + MP - 1) / MP;
    const bool mfast = mtiles <= 4;
    const int mtile = mfast ? lin % mtiles : lin / nblocks;
    const int nblock = mfast ? lin / mtiles : lin % nblocks;
    const int m0 = mtile * MP, nt0 = nblock * NTT;
    const int nck = a.kchunks;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.xq, uint32_t(int64_t(a.M) * a.Kp));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, a.s_bytes);
    const uint32_t s_shift = 16u * (c & 1);

    f32x4 acc[MTW][NTW];
    i32x4 tmp[MTW][NTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            tmp[i][j] = i32x4{0, 0, 0, 0};
        }

    auto xswz = [](int r) { return P == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
    auto slot = [&](int r, int p) { return (r / RPI) * 1024 + ((r % RPI) * P + (p ^ xswz(r))) * 16; };

    uint32_t a_off[NAW];
#pragma unroll
    for (int q = 0; q < NAW; ++q) {
        const int row = ((wv + W * q) % NA) * RPI + lane / P;
        const int m = m0 + row;
        const uint32_t kb = 16u * uint32_t((lane % P) ^ xswz(row));
        a_off[q] = (m < a.M) ? uint32_t(m) * uint32_t(a.Kp) + kb : 0x80000000u;
    }
    uint32_t b_off[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q)
        b_off[q] = uint32_t(nt0 + (wv + W * q) % NB) * uint32_t(a.kchunks) * TILE_BYTES + uint32_t(lane) * 16u;
    int s_tile[NSS], s_q[NSS], s_w[NSS];
#pragma unroll
    for (int d = 0; d < NSS; ++d) {
        const int e = d * 64 + lane;
        s_tile[d] = e / (8 * SPC);
        s_q[d] = (e / 8) % SPC;
        s_w[d] = e % 8;
    }
    auto group_of = [&](int kc, int q) -> uint32_t {
        return (GS <= STEPS) ? uint32_t(kc * (STEPS / GS) + q) : uint32_t(kc / (GS / STEPS));
    };

    auto issue = [&](int kc, int buf) {
        uint8_t *base = lds + buf * STAGE;
#pragma unroll
        for (int q = 0; q < NAW; ++q) ld128_lds(xr, a_off[q] + uint32_t(kc) * CH, base + ((wv + W * q) % NA) * 1024);
#pragma unroll
        for (int q = 0; q < NBW; ++q)
            ld128_lds(wr, b_off[q] + uint32_t(kc) * TILE_BYTES, base + A_BYTES + ((wv + W * q) % NB) * 1024);
        uint8_t *sc = base + A_BYTES + B_BYTES + wv * SCW;
#pragma unroll
        for (int d = 0; d < NSS; ++d) {
            const uint32_t ntg = uint32_t(nt0 + wn * NTW + s_tile[d]);
            uint32_t off = (ntg * uint32_t(a.ngroups) + group_of(kc, s_q[d])) * (TILE_N * 2) + uint32_t(s_w[d]) * 4;
            if (s_tile[d] >= NTW) off = 0x80000000u;
            ld32_lds(sr, off, sc + d * 256);
        }
    };

    auto compute = [&](int kc, int buf) {
        const uint8_t *A = lds + buf * STAGE;
        const uint8_t *Bt = A + A_BYTES;
        const uint8_t *sc = A + A_BYTES + B_BYTES + wv * SCW;
        u32x4 wq[NTW];
        uint32_t sq[NTW][SPC];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            wq[j] = *reinterpret_cast<const u32x4 *>(Bt + (wn * NTW + j) * 1024 + lane * 16);
#pragma unroll
            for (int q = 0; q < SPC; ++q)
                sq[j][q] = *reinterpret_cast<const uint32_t *>(sc + ((j * SPC + q) * 8 + (c >> 1)) * 4);
        }
#pragma unroll
        for (int st = 0; st < ST8; ++st) {
            i32x4 af[MTW];
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
                af[mt] = *reinterpret_cast<const i32x4 *>(A + slot((wm * MTW + mt) * 16 + c, 4 * st + g));
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const i32x4 bv = b_operand<WF>(wq[j], st);
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt)
                    tmp[mt][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bv, tmp[mt][j], 0, 0, 0);
            }
            // fold the exact group sums at the group's last step (a group may span chunks)
            bool boundary;
            if (GS <= STEPS) boundary = ((2 * st + 2) % GS) == 0;
            else boundary = (st == ST8 - 1) && (((kc + 1) % (GS / STEPS)) == 0);
            if (boundary) {
                const int q = (GS <= STEPS) ? (2 * st) / GS : 0;
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const uint32_t sbits = (sq[j][q] >> s_shift) & 0xFFFFu;
                    const float sg = WF == FMT_INT4 ? f16_bits_to_f32(sbits) : bf16_bits_to_f32(sbits);
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][j][r] = fmaf(sg, float(tmp[mt][j][r]), acc[mt][j][r]);
                        tmp[mt][j] = i32x4{0, 0, 0, 0};
                    }
                }
            }
        }
    };

#pragma unroll
    for (int u = 0; u < S - 1; ++u)
        if (u < nck) issue(u, u);
    for (int i0 = 0; i0 < nck; i0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int i = i0 + u;
            if (i < nck) {
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

    // ---- epilogue: row scale, bias, output rounding ----
    const int es = a.out_f32 ? 4 : 2;
    if (m0 + MP <= a.M && (nt0 + NTT) * TILE_N <= a.N &&
        uint64_t(MP) * uint64_t(a.N) * uint64_t(es) < (uint64_t(1) << 32)) {
        // a tile wholly inside the output: one ranged buffer for its rows, each store = lane
        // offset + wave-uniform row offset + column-tile immediate; type and bias chosen once
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
                    const int rl = (wm * MTW + mt) * 16 + r;             // row within the tile, lane row g*4 on top
                    const uint32_t row_off = uint32_t(rl) * uint32_t(a.N) * ES;
                    const float rsc = a.xs[m0 + rl + g * 4];
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        // the same expression as the checked path below
                        const float v = BIAS ? fmaf(acc[mt][j][r], rsc, bj[j]) : acc[mt][j][r] * rsc;
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
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + (wm * MTW + mt) * 16 + g * 4 + r;
            if (m >= a.M) continue;
            const float rs = a.xs[m];
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int n = (nt0 + wn * NTW + j) * TILE_N + c;
                if (n >= a.N) continue;
                // row scale and bias: one fused multiply-add when there is a bias
                const float v = a.bias ? fmaf(acc[mt][j][r], rs, bf16_bits_to_f32(a.bias[n])) : acc[mt][j][r] * rs;
                if (a.out_f32) reinterpret_cast<float *>(a.out)[int64_t(m) * a.N + n] = v;
                else reinterpret_cast<__bf16 *>(a.out)[int64_t(m) * a.N + n] = (__bf16)v;
            }
        }
}

// stage bytes and ring depth of an INT8-compute schedule
constexpr int a8_stage_bytes(int wf, int gs, int wm, int wn, int mt, int nt) {
    return 16 * mt * wm * chunk_k(wf) + nt * wn * TILE_BYTES + wm * wn * 256 * gemv_scale_blocks(wf, gs, nt);
}
constexpr int a8_depth(int wf, int gs, int wm, int wn, int mt, int nt) {
    const int d = LDS_BYTES_MAX / a8_stage_bytes(wf, gs, wm, wn, mt, nt);
    return d > 6 ? 6 : d;
}

template <int WF, int GS, int I>
hipError_t launch_a8_one(const A8Args &a, hipStream_t st) {
    constexpr A8Tile t = A8_TILES[I];
    constexpr int depth = a8_depth(WF, GS, t.WM, t.WN, t.MT, t.NT);
    static_assert(depth >= 2, "two stages fit the LDS");
    constexpr size_t lds = size_t(depth) * a8_stage_bytes(WF, GS, t.WM, t.WN, t.MT, t.NT);
    auto kern = qgemm_a8_kernel<WF, GS, t.WM, t.WN, t.MT, t.NT, depth>;
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(lds));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int MP = 16 * t.MT * t.WM, NTT = t.NT * t.WN;
    const int blocks = int(ceil_div(a.M, MP) * ceil_div(a.ntiles, NTT));
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * t.WM * t.WN), lds, st, a);
    return hipGetLastError();
}

template <int WF, int GS>
hipError_t launch_a8_gs(int tile, const A8Args &a, hipStream_t st) {
    static_assert(NUM_A8_TILES == 5, "one case per compiled schedule");
    switch (tile) {
        case 0: return launch_a8_one<WF, GS, 0>(a, st);
        case 1: return launch_a8_one<WF, GS, 1>(a, st);
        case 2: return launch_a8_one<WF, GS, 2>(a, st);
        case 3: return launch_a8_one<WF, GS, 3>(a, st);
        default: return launch_a8_one<WF, GS, 4>(a, st);
    }
}

template <int WF>
hipError_t launch_a8_wf(int gs, int tile, const A8Args &a, hipStream_t st) {
    switch (gs) {
        case 2: return launch_a8_gs<WF, 2>(tile, a, st);
        case 4: return launch_a8_gs<WF, 4>(tile, a, st);
        default: return launch_a8_gs<WF, 8>(tile, a, st);
    }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t *x, int M, int K, int Kp, int layout, int8_t *codes, float *scales,
                            hipStream_t st) {
    const dim3 grid(M);
    if (layout == 0)
        hipLaunchKernelGGL(quant_act_kernel<0>, grid, dim3(256), 0, st, x, M, K, Kp, codes, scales);
    else if (layout == 1)
        hipLaunchKernelGGL(quant_act_kernel<1>, grid, dim3(256), 0, st, x, M, K, Kp, codes, scales);
    else
        hipLaunchKernelGGL(quant_act_kernel<2>, grid, dim3(256), 0, st, x, M, K, Kp, codes, scales);
    return hipGetLastError();
}

hipError_t launch_gemm_a8(const Layout &L, int tile, const uint16_t *x, int M, const void *pw, const void *ps,
                          const void *bias, void *out, bool out_f32, int8_t *xq, float *xs, hipStream_t st) {
    const int Kp = int(L.Kp);
    hipError_t e = launch_quant_act(x, M, int(L.K), Kp, L.fmt == FMT_INT4 ? 1 : 2, xq, xs, st);
    if (e != hipSuccess) return e;
    A8Args a{};
    a.xq = xq;
    a.xs = xs;
    a.w = static_cast<const uint8_t *>(pw);
    a.s = static_cast<const uint8_t *>(ps);
    a.M = M;
    a.N = int(L.N);
    a.Kp = Kp;
    a.kchunks = int(L.kchunks);
    a.ngroups = int(L.ngroups);
    a.ntiles = int(L.ntiles);
    a.out_f32 = out_f32 ? 1 : 0;
    a.bias = static_cast<const uint16_t *>(bias);
    a.out = out;
    a.w_bytes = uint32_t(L.w_bytes);
    a.s_bytes = uint32_t(L.s_bytes);
    return (L.fmt == FMT_INT4) ? launch_a8_wf<FMT_INT4>(L.group / 32, tile, a, st)
                               : launch_a8_wf<FMT_INT8>(L.group / 32, tile, a, st);
}

}  // namespace ql
