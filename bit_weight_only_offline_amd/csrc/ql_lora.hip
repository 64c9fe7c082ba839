// In-place low-rank update of a packed INT8 weight, requantised into the same buffers:
//     W <- beta * D(W) + alpha * (mat1 @ mat2)
// (piper-kernels package description, "ConvRot INT8": addmm_ follows the Tensor.addmm_
// contract, requantises and keeps the quantised storage; an unsigned 64-bit rounding seed
// picks one of the two neighbouring INT8 codes at random with probability set by the
// distance, leaves the deterministic scales alone and uses no global generator).
//
// Arithmetic, IEEE float32 with one rounding per operation (contraction off outside the
// explicit fused multiply-adds), so that every code and scale is the unique one the
// definition gives:
//   w_old = q * s                                  (exact: 8-bit code times bf16 scale)
//   d_0 = +0,  d_j = fma(mat1[n, j], mat2[j, k], d_{j-1})   in index order
//   w     = beta * w_old + alpha * d               (two products, then their sum)
//   s'    = bf16(amax_group |w| / 127)             (the RTN scale rule of the quantiser)
//   v     = w / s',  code = clamp(rint(v), -127, 127)            without a seed
//                    code = clamp(floor(v) + [u < v - floor(v)], -127, 127)   with one
// u is the top 24 bits of SplitMix64 output n*K + k of the seed, times 2^-24.  SplitMix64
// (Steele, Lea and Flood, OOPSLA 2014): output i is the 64-bit finaliser (Stafford's
// variant 13) of seed + (i + 1) * 0x9E3779B97F4A7C15.  A scale that rounds to zero gives
// codes 0.
//
// Layout: the packed INT8 weight is 1 KiB tiles [column tile][64-input chunk]; lane l of
// a tile holds column l % 16 and inputs 8 (l / 16) .. +7 of both 32-wide k-steps, stored
// offset-binary (q ^ 0x80).  Scales are [column tile][group][16] bf16.
//
// One workgroup owns 256 consecutive inputs (four chunks, one thread per input) of a run
// of column tiles.  Per tile it stages the 4 KiB of codes through LDS, transposed to
// [input][column], so that each thread then holds its input's 16 codes, one per column;
// the low-rank product runs with the adapter's row n as a wave-uniform operand and mat2's
// column k in registers; a group's amax is a lane-shuffle reduction (and a cross-wave
// one through LDS for groups of 128 and 256 inputs); the new codes go back through the
// same LDS transpose and are stored over the old ones.  Each code and scale is read and
// written by the same thread, so the update is safe in place.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "ql_common.hpp"
#include "ql_decode.hpp"
#include "ql_launch.hpp"

namespace ql {
namespace {

constexpr int LM_KB = 256;        // inputs per workgroup, one per thread
constexpr int LM_MAX_RANK = 256;  // adapter rank limit (its rows of one tile sit in LDS)

__device__ inline uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// max over each row of 16 lanes, left in every lane of the row (DPP: swap neighbours,
// swap pairs, mirror the half-rows, mirror the row); the values are non-negative float32
// bit patterns, whose order as unsigned integers is their order as numbers
__device__ inline uint32_t row_max16(uint32_t v) {
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false)));    // quad_perm 1,0,3,2
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false)));    // quad_perm 2,3,0,1
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false)));   // row_half_mirror
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false)));   // row_mirror
    return v;
}

__device__ inline uint32_t lane_value(uint32_t v, int l) { return uint32_t(__builtin_amdgcn_readlane(int(v), l)); }

constexpr int LM_ROW = LM_KB + 32;   // LDS row stride of the code transpose (bytes)

// G: group size (32 .. 256); RR: rank chunk held in registers (8, 16, 32 or 64; the rank
// runs in chunks of RR, zero-padded past the real rank: adding +-0 changes no sum here,
// since a running sum that starts at +0 is never -0)
template <int G, int RR>
__global__ void __launch_bounds__(256) lora_merge8_kernel(uint8_t *__restrict__ w, uint16_t *__restrict__ s,
                                                          const uint16_t *__restrict__ m1,
                                                          const uint16_t *__restrict__ m2, int N, int K, int rank,
                                                          int kchunks, int ngp, int ntiles, int tiles_per_wg,
                                                          float alpha, float beta, int stochastic, uint64_t seed) {
#pragma clang fp contract(off)
    __shared__ __align__(16) uint8_t T[16 * LM_ROW];      // [column][input] codes of one tile
    __shared__ uint32_t red[4][16];                       // per-wave amax (groups over 64)
    __shared__ __align__(16) float M1[LM_MAX_RANK * 16];  // mat1 rows of the tile [chunk][column][RR]
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int kc = blockIdx.x * 4 + wv;                   // this wave's chunk
    const bool chunk_ok = kc < kchunks;
    const int k = blockIdx.x * LM_KB + t;                 // this thread's input
    const bool k_ok = k < K;
    const int grp = k / G;
    const int nt0 = blockIdx.y * tiles_per_wg;
    const int nt1 = min(ntiles, nt0 + tiles_per_wg);
    const int nrch = (rank + RR - 1) / RR;
    const int rg = lane >> 4, rc = lane & 15;             // this thread's packed record: lane (rg, rc)
    const int half = lane >> 5;                           // groups of 32: two per wavefront

    float m2v[RR];
    for (int nt = nt0; nt < nt1; ++nt) {
        // ---- stage: packed records -> [column][input]; mat1 rows -> LDS ----
        const int64_t rec_off = ((int64_t(nt) * kchunks + kc) * 64 + lane) * 16;
        u32x4 rec = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
        if (chunk_ok) rec = *reinterpret_cast<const u32x4 *>(w + rec_off);
        uint8_t *trow = T + rc * LM_ROW + wv * 64 + 8 * rg;
        *reinterpret_cast<u32x2 *>(trow) = u32x2{rec[0], rec[1]};          // inputs 8 rg .. +7
        *reinterpret_cast<u32x2 *>(trow + 32) = u32x2{rec[2], rec[3]};     // inputs 32 + 8 rg .. +7
        for (int e = t; e < nrch * 16 * RR; e += 256) {
            const int jj = e % RR, c = (e / RR) % 16, j = (e / (16 * RR)) * RR + jj;
            const int n = nt * TILE_N + c;
            M1[e] = (n < N && j < rank) ? bf16_to_f32(m1[int64_t(n) * rank + j]) : 0.0f;
        }
        __syncthreads();
        uint32_t qb[16];                                   // offset-binary codes at input k
#pragma unroll
        for (int c = 0; c < 16; ++c) qb[c] = T[c * LM_ROW + t];

        // ---- old scales of this input's group, one per column ----
        float so[16];
        {
            u32x4 s0 = {0u, 0u, 0u, 0u}, s1 = {0u, 0u, 0u, 0u};
            if (chunk_ok) {
                const u32x4 *sp = reinterpret_cast<const u32x4 *>(s + (int64_t(nt) * ngp + grp) * 16);
                s0 = sp[0];
                s1 = sp[1];
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                so[c] = bf16_to_f32(uint16_t(s0[c >> 1] >> (16 * (c & 1))));
                so[8 + c] = bf16_to_f32(uint16_t(s1[c >> 1] >> (16 * (c & 1))));
            }
        }

        // ---- d = mat1 @ mat2 for the 16 columns at input k: fused multiply-adds in index order ----
        float acc[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[c] = 0.0f;
        for (int ch = 0; ch < nrch; ++ch) {
            if (nrch > 1 || nt == nt0) {
                const int kk = k_ok ? k : K - 1;
#pragma unroll
                for (int jj = 0; jj < RR; ++jj) {
                    const int j = ch * RR + jj;
                    const float v = bf16_to_f32(m2[int64_t(j < rank ? j : rank - 1) * K + kk]);
                    m2v[jj] = (k_ok && j < rank) ? v : 0.0f;
                }
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float *row = M1 + (ch * 16 + c) * RR;     // the same address in every lane
#pragma unroll
                for (int jj = 0; jj < RR; ++jj) acc[c] = __builtin_fmaf(row[jj], m2v[jj], acc[c]);
            }
        }

        // ---- merged weights and each group's amax ----
        float wn[16];
        uint32_t am[16];                                  // |w| maxima as float32 bits
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float w_old = float(int(qb[c]) - 128) * so[c];
            const float t1 = beta * w_old;
            const float t2 = alpha * acc[c];
            wn[c] = t1 + t2;
            const uint32_t r = row_max16(__float_as_uint(fabsf(wn[c])));
            const uint32_t r0 = lane_value(r, 0), r1 = lane_value(r, 16), r2 = lane_value(r, 32),
                           r3 = lane_value(r, 48);
            am[c] = G == 32 ? (half ? max(r2, r3) : max(r0, r1)) : max(max(r0, r1), max(r2, r3));
        }
        if (G > 64) {
            if (lane == 0) {
#pragma unroll
                for (int c = 0; c < 16; ++c) red[wv][c] = am[c];
            }
            __syncthreads();
            constexpr int WPG = G / 64;                   // waves per group
            const int w0 = (wv / WPG) * WPG;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                uint32_t m = red[w0][c];
#pragma unroll
                for (int i = 1; i < WPG; ++i) m = max(m, red[w0 + i][c]);
                am[c] = m;
            }
        }

        // ---- new scales: lane c (and 32 + c) divides for column c, then all read them ----
        uint32_t my = am[0];
#pragma unroll
        for (int c = 1; c < 16; ++c) my = rc == c ? am[c] : my;
        const __bf16 my_s = (__bf16)__fdiv_rn(__uint_as_float(my), 127.0f);
        const uint32_t my_bits = __builtin_bit_cast(uint16_t, my_s);
        uint32_t sb[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const uint32_t lo_b = lane_value(my_bits, c);
            sb[c] = G == 32 ? (half ? lane_value(my_bits, 32 + c) : lo_b) : lo_b;
        }

        // ---- requantise ----
        const uint64_t ctr0 = uint64_t(nt) * TILE_N * uint64_t(K) + uint64_t(k);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float sn = bf16_to_f32(uint16_t(sb[c]));
            float qf = 0.0f;
            if (sn > 0.0f) {
                const float v = __fdiv_rn(wn[c], sn);
                if (stochastic) {
                    const float lo = floorf(v);
                    const float dist = v - lo;
                    const uint64_t z = splitmix64_at(seed, ctr0 + uint64_t(c) * uint64_t(K));
                    // u < dist with u = (z >> 40) 2^-24, both sides scaled by 2^24 (exact)
                    qf = float(uint32_t(z >> 40)) < dist * 16777216.0f ? lo + 1.0f : lo;
                } else {
                    qf = rintf(v);
                }
                qf = fminf(fmaxf(qf, -127.0f), 127.0f);
            }
            T[c * LM_ROW + t] = uint8_t(int(qf) + 128);
        }
        if (chunk_ok && (k % G) == 0) {
            u32x4 *sp = reinterpret_cast<u32x4 *>(s + (int64_t(nt) * ngp + grp) * 16);
            sp[0] = u32x4{sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16), sb[4] | (sb[5] << 16), sb[6] | (sb[7] << 16)};
            sp[1] = u32x4{sb[8] | (sb[9] << 16), sb[10] | (sb[11] << 16), sb[12] | (sb[13] << 16),
                          sb[14] | (sb[15] << 16)};
        }
        __syncthreads();

        // ---- [column][input] -> packed record, stored over the old one ----
        const u32x2 lo8 = *reinterpret_cast<const u32x2 *>(trow);
        const u32x2 hi8 = *reinterpret_cast<const u32x2 *>(trow + 32);
        if (chunk_ok) *reinterpret_cast<u32x4 *>(w + rec_off) = u32x4{lo8.x, lo8.y, hi8.x, hi8.y};
        __syncthreads();
    }
}

template <int G>
hipError_t launch_g(dim3 grid, uint8_t *w, uint16_t *s, const uint16_t *m1, const uint16_t *m2, int N, int K,
                    int rank, int kchunks, int ngp, int ntiles, int tpw, float alpha, float beta, int stochastic,
                    uint64_t seed, hipStream_t st) {
    if (rank <= 8)
        hipLaunchKernelGGL((lora_merge8_kernel<G, 8>), grid, dim3(256), 0, st, w, s, m1, m2, N, K, rank, kchunks,
                           ngp, ntiles, tpw, alpha, beta, stochastic, seed);
    else if (rank <= 16)
        hipLaunchKernelGGL((lora_merge8_kernel<G, 16>), grid, dim3(256), 0, st, w, s, m1, m2, N, K, rank, kchunks,
                           ngp, ntiles, tpw, alpha, beta, stochastic, seed);
    else if (rank <= 32)
        hipLaunchKernelGGL((lora_merge8_kernel<G, 32>), grid, dim3(256), 0, st, w, s, m1, m2, N, K, rank, kchunks,
                           ngp, ntiles, tpw, alpha, beta, stochastic, seed);
    else
        hipLaunchKernelGGL((lora_merge8_kernel<G, 64>), grid, dim3(256), 0, st, w, s, m1, m2, N, K, rank, kchunks,
                           ngp, ntiles, tpw, alpha, beta, stochastic, seed);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lora_merge8(const Layout &L, void *pw, void *ps, const void *mat1, const void *mat2, int rank,
                              float alpha, float beta, int stochastic, uint64_t seed, hipStream_t st) {
    const int kchunks = int(L.kchunks), ntiles = int(L.ntiles), ngp = int(L.ngroups);
    const int gx = (kchunks + 3) / 4;
    // a run of column tiles per workgroup (mat2's columns stay in registers across it),
    // with about 2048 workgroups in flight over the whole weight
    const int64_t units = int64_t(gx) * ntiles;
    const int tpw = int(std::min<int64_t>(32, std::max<int64_t>(1, units / 2048)));
    const dim3 grid(gx, (ntiles + tpw - 1) / tpw);
    uint8_t *w = static_cast<uint8_t *>(pw);
    uint16_t *s = static_cast<uint16_t *>(ps);
    const uint16_t *m1 = static_cast<const uint16_t *>(mat1), *m2 = static_cast<const uint16_t *>(mat2);
    const int N = int(L.N), K = int(L.K);
    switch (L.group) {
        case 32: return launch_g<32>(grid, w, s, m1, m2, N, K, rank, kchunks, ngp, ntiles, tpw, alpha, beta,
                                     stochastic, seed, st);
        case 64: return launch_g<64>(grid, w, s, m1, m2, N, K, rank, kchunks, ngp, ntiles, tpw, alpha, beta,
                                     stochastic, seed, st);
        case 128: return launch_g<128>(grid, w, s, m1, m2, N, K, rank, kchunks, ngp, ntiles, tpw, alpha, beta,
                                       stochastic, seed, st);
        default: return launch_g<256>(grid, w, s, m1, m2, N, K, rank, kchunks, ngp, ntiles, tpw, alpha, beta,
                                      stochastic, seed, st);
    }
}

}  // namespace ql
