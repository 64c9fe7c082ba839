// On-device round-to-nearest quantiser: dense float32 weights [N, K] -> the canonical
// arrays that qlinear_pack() consumes.
//
// This is the step before the offline pack: quantising a dense high-precision weight
// (piper-kernels package description, "ConvRot INT8": from_hp with group_size=256) with
// the round-to-nearest rules of the offline packer in selective_state_update_pairnib.py
// (pack_pairnib: per-group amax, scale, rint to the grid).  Every number is IEEE float32
// with round-to-nearest-even per operation, in the same order as the definition, so the
// codes and scales are the unique ones the rules give:
//   INT4 symmetric   s = fp16(amax / 7),  q = clamp(rint(w / s), -8, 7)
//   INT4 asymmetric  lo = min(min w, 0), hi = max(max w, 0), s = fp16((hi - lo) / 15),
//                    z = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15)
//   INT8             s = bf16(amax / 127), q = clamp(rint(w / s), -127, 127)
//   MXFP4            e = floor(log2 amax) - 2 clamped to [-127, 127] (0 for an all-zero
//                    block), element = nearest E2M1 value of w * 2^-e, ties to the even
//                    code, saturating at 6, no negative zero; scale code e + 127
//   codebook         norm = bf16 of the exact row norm (the exact sum of the squares,
//                    one correctly rounded bf16 square root, ties to even),
//                    u = (w * fp32(sqrt K)) / norm, index = nearest level (distances in
//                    float64), ties to the lower index
// A scale that rounds to zero gives codes 0 (and zero-point 0).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "ql_common.hpp"
#include "ql_launch.hpp"

namespace ql {
namespace {

// reductions over aligned runs of W lanes (W a power of two <= 64; every lane of the
// wavefront takes part)
template <int W>
__device__ inline float seg_max(float v) {
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
template <int W>
__device__ inline float seg_min(float v) {
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
    return v;
}

// E2M1 magnitude code of a >= 0: nearest of 0, .5, 1, 1.5, 2, 3, 4, 6; a tie goes to
// the even code, values above 6 saturate
__device__ inline uint32_t e2m1_mag(float a) {
    if (a <= 0.25f) return 0;
    if (a < 0.75f) return 1;
    if (a <= 1.25f) return 2;
    if (a < 1.75f) return 3;
    if (a <= 2.5f) return 4;
    if (a < 3.5f) return 5;
    if (a <= 5.0f) return 6;
    return 7;
}

// A wavefront quantises 64 / PL groups side by side: a group of G = 2 * PG elements is
// held by PL = min(PG, 64) lanes, each with PG / PL element pairs (8-byte loads,
// coalesced along the row).  PG = G / 2 is a template parameter (16 .. 128).
template <int FMT, bool ZP, int PG>
__global__ void __launch_bounds__(256) quant_group_kernel(const float *__restrict__ w, int N, int K,
                                                          uint8_t *__restrict__ codes, void *__restrict__ scales,
                                                          uint8_t *__restrict__ zeros) {
    constexpr int G = 2 * PG;
    constexpr int PL = PG < 64 ? PG : 64;                // lanes per group
    constexpr int PPL = PG / PL;                         // pairs per lane
    constexpr int GPW = 64 / PL;                         // groups per wavefront
    const int lane = threadIdx.x & 63;
    const int sub = lane % PL;
    const int ng = K / G;
    const int64_t gid = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * GPW + lane / PL;
    const bool live = gid < int64_t(N) * ng;             // lanes past the last group idle
    const int64_t n = live ? gid / ng : 0;
    const int gq = live ? int(gid % ng) : 0;
    const int64_t base = n * int64_t(K) + int64_t(gq) * G;

    float2 v[PPL];
#pragma unroll
    for (int j = 0; j < PPL; ++j)
        v[j] = live ? *reinterpret_cast<const float2 *>(w + base + 2 * (sub + PL * j)) : float2{0.0f, 0.0f};
    auto pair_index = [&](int j) { return base / 2 + sub + PL * j; };

    if (FMT == FMT_INT4 && ZP) {
        float mn = 0.0f, mx = 0.0f;                      // lo = min(min w, 0), hi = max(max w, 0)
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            mn = fminf(mn, fminf(v[j].x, v[j].y));
            mx = fmaxf(mx, fmaxf(v[j].x, v[j].y));
        }
        const float lo = seg_min<PL>(mn), hi = seg_max<PL>(mx);
        if (!live) return;
        const _Float16 s16 = (_Float16)__fdiv_rn(__fsub_rn(hi, lo), 15.0f);
        const float s = (float)s16;
        const bool ok = s > 0.0f;
        const float z = ok ? fminf(fmaxf(rintf(__fdiv_rn(-lo, s)), 0.0f), 15.0f) : 0.0f;
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            uint32_t q0 = 0, q1 = 0;
            if (ok) {
                q0 = uint32_t(fminf(fmaxf(__fadd_rn(rintf(__fdiv_rn(v[j].x, s)), z), 0.0f), 15.0f));
                q1 = uint32_t(fminf(fmaxf(__fadd_rn(rintf(__fdiv_rn(v[j].y, s)), z), 0.0f), 15.0f));
            }
            codes[pair_index(j)] = uint8_t(q0 | (q1 << 4));
        }
        if (sub == 0) {
            reinterpret_cast<_Float16 *>(scales)[gid] = s16;
            zeros[gid] = uint8_t(z);
        }
        return;
    }

    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < PPL; ++j) amax = fmaxf(amax, fmaxf(fabsf(v[j].x), fabsf(v[j].y)));
    amax = seg_max<PL>(amax);
    if (!live) return;

    if (FMT == FMT_INT4) {
        const _Float16 s16 = (_Float16)__fdiv_rn(amax, 7.0f);
        const float s = (float)s16;
        const bool ok = s > 0.0f;
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            int32_t q0 = 0, q1 = 0;
            if (ok) {
                q0 = int32_t(fminf(fmaxf(rintf(__fdiv_rn(v[j].x, s)), -8.0f), 7.0f));
                q1 = int32_t(fminf(fmaxf(rintf(__fdiv_rn(v[j].y, s)), -8.0f), 7.0f));
            }
            codes[pair_index(j)] = uint8_t((q0 & 15) | ((q1 & 15) << 4));   // two's complement nibbles
        }
        if (sub == 0) reinterpret_cast<_Float16 *>(scales)[gid] = s16;
    } else if (FMT == FMT_INT8) {
        const __bf16 sb = (__bf16)__fdiv_rn(amax, 127.0f);
        const float s = (float)sb;
        const bool ok = s > 0.0f;
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            int32_t q0 = 0, q1 = 0;
            if (ok) {
                q0 = int32_t(fminf(fmaxf(rintf(__fdiv_rn(v[j].x, s)), -127.0f), 127.0f));
                q1 = int32_t(fminf(fmaxf(rintf(__fdiv_rn(v[j].y, s)), -127.0f), 127.0f));
            }
            reinterpret_cast<uint16_t *>(codes)[pair_index(j)] = uint16_t((q0 & 0xFF) | ((q1 & 0xFF) << 8));
        }
        if (sub == 0) reinterpret_cast<__bf16 *>(scales)[gid] = sb;
    } else {   // MXFP4
        int e = 0;
        if (amax > 0.0f) {
            int ex;
            frexpf(amax, &ex);                           // amax = m 2^ex, m in [0.5, 1)
            e = min(max(ex - 3, -127), 127);             // floor(log2 amax) - 2
        }
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            const float a0 = ldexpf(v[j].x, -e), a1 = ldexpf(v[j].y, -e);   // power-of-two scaling
            uint32_t m0 = e2m1_mag(fabsf(a0)), m1 = e2m1_mag(fabsf(a1));
            if (a0 < 0.0f && m0 != 0) m0 |= 8;
            if (a1 < 0.0f && m1 != 0) m1 |= 8;
            codes[pair_index(j)] = uint8_t(m0 | (m1 << 4));
        }
        if (sub == 0) reinterpret_cast<uint8_t *>(scales)[gid] = uint8_t(e + 127);
    }
}

struct Levels { float c[16]; };

// float64 -> bf16, one rounding to 8 significant bits with ties to even (the spacing
// stops shrinking below the float32 normal range); finite non-negative input
__host__ __device__ inline float bf16_from_double(double a) {
    if (!(a > 0.0)) return 0.0f;
    int e;
    frexp(a, &e);                                        // a in [2^(e-1), 2^e)
    const int q = (e > -125 ? e : -125) - 8;
    return (float)ldexp(rint(ldexp(a, -q)), q);
}

// ---- exact sum of float32 squares --------------------------------------------------------
// A float32 |w| = m * 2^(f - 150) with m < 2^24 and f = max(biased exponent, 1), so
// w^2 = m^2 * 2^(2f - 300) with m^2 < 2^48.  Relative to the row's largest f (F), the
// squares are summed as integers on a 320-bit grid (five 64-bit limbs) whose unit is
// 2^(2F - 300 - SQ_SHIFT): the largest square sits at bits 241..288, and 2^30 of them
// stay below bit 319.  Bits of a square that fall below the grid only set a sticky flag
// (the sum is then strictly above the grid value).  Integer addition is associative, so
// the result does not depend on the order of the additions.
constexpr int SQ_SHIFT = 241;
struct Sum320 {
    uint64_t l[5];
    uint32_t sticky;
};

__host__ __device__ inline void add320(Sum320 &a, const Sum320 &b) {
    uint64_t c = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const uint64_t t = a.l[i] + c;
        const uint64_t c1 = t < c;
        a.l[i] = t + b.l[i];
        c = c1 + (a.l[i] < t);
    }
    a.sticky |= b.sticky;
}

// add v * 2^shift (v < 2^48) to the accumulator; shift <= SQ_SHIFT
__host__ __device__ inline void add_shifted(Sum320 &a, uint64_t v, int shift) {
    if (shift < 0) {
        const int d = -shift;
        if (d >= 48) {
            a.sticky |= v != 0;
            return;
        }
        a.sticky |= (v & ((uint64_t(1) << d) - 1)) != 0;
        v >>= d;
        shift = 0;
    }
    const int q = shift >> 6, r = shift & 63;
    const uint64_t lo = v << r, hi = r ? (v >> (64 - r)) : 0;
    uint64_t c = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const uint64_t add = (i == q) ? lo : ((i == q + 1) ? hi : 0);
        const uint64_t t = a.l[i] + c;
        const uint64_t c1 = t < c;
        a.l[i] = t + add;
        c = c1 + (a.l[i] < t);
    }
}

// sign of (sum - v) for a double v > 0 with at most 18 significant bits on the grid
// of unit 2^unit_exp; v's bits at or above the unit (the caller keeps them there)
__host__ __device__ inline int cmp_sum(const Sum320 &a, double v, int unit_exp) {
    int e;
    const double f = frexp(v, &e);                       // v = f * 2^e, f in [0.5, 1)
    const uint64_t mv = uint64_t(ldexp(f, 18));          // exact: v has <= 18 bits
    const int sh = e - 18 - unit_exp;                    // v = mv * 2^sh units
    if (sh > 320 - 18) return -1;                        // v >= 2^319 units: above any sum
    // The midpoints compared lie within a few bf16 steps of sqrt(sum), whose square is at
    // least the largest square (>= 2^(2F - 300) x 2^46 for a normal F, the whole grid
    // below it being 2^(SQ_SHIFT - 46) units): their 18-bit squares sit far above the
    // unit, so sh >= 0 for every comparison made.  A v off the grid (sh < 0) is compared
    // by its integer part, ties above.
    Sum320 b = {{0, 0, 0, 0, 0}, 0};
    add_shifted(b, sh >= 0 ? mv : (mv >> (-sh < 63 ? -sh : 63)), (sh > 0 ? sh : 0));
#pragma unroll
    for (int i = 4; i >= 0; --i) {
        if (a.l[i] != b.l[i]) return a.l[i] > b.l[i] ? 1 : -1;
    }
    return a.sticky ? 1 : (sh >= 0 ? 0 : -1);
}

// value of a non-negative bf16 pattern; the infinity stands for 2^128, so that its
// midpoint with the largest finite value is the overflow threshold of rounding
__host__ __device__ inline double bf16_pattern_value(uint32_t b) {
    return b >= 0x7F80u ? ldexp(1.0, 128) : (double)__builtin_bit_cast(float, uint32_t(b << 16));
}

// bf16 nearest to sqrt(sum), ties to even: the answer is the bf16 value b whose
// midpoints with its neighbours bracket sqrt(sum), decided by comparing the exact sum
// with the midpoints' squares (9-bit midpoints: their squares are exact doubles)
__host__ __device__ inline float bf16_sqrt_of_sum(const Sum320 &a, int unit_exp) {
    int top = -1;
#pragma unroll
    for (int i = 4; i >= 0; --i)
        if (top < 0 && a.l[i] != 0) top = i;
    if (top < 0) return 0.0f;                            // every square is 0
    double approx = ldexp((double)a.l[top], 64 * top + unit_exp);
    if (top > 0) approx += ldexp((double)a.l[top - 1], 64 * (top - 1) + unit_exp);
    uint32_t b = __builtin_bit_cast(uint32_t, bf16_from_double(sqrt(approx))) >> 16;
    for (int it = 0; it < 8; ++it) {
        const uint32_t hi = b >= 0x7F80u ? 0x7F80u : b + 1;
        const double mhi = 0.5 * (bf16_pattern_value(b) + bf16_pattern_value(hi));
        const double mlo = b == 0 ? 0.0 : 0.5 * (bf16_pattern_value(b - 1) + bf16_pattern_value(b));
        const int c_hi = b >= 0x7F80u ? -1 : cmp_sum(a, mhi * mhi, unit_exp);
        const int c_lo = b == 0 ? 1 : cmp_sum(a, mlo * mlo, unit_exp);
        if (c_hi > 0 || (c_hi == 0 && (b & 1u))) b = hi;
        else if (c_lo < 0 || (c_lo == 0 && (b & 1u))) b = b - 1;
        else break;
    }
    return b >= 0x7F80u ? __builtin_bit_cast(float, 0x7F800000u) : __builtin_bit_cast(float, uint32_t(b << 16));
}

// One workgroup (256 threads) per row: the row's largest exponent, the exact sum of the
// squares (per thread, then a fixed-order tree of exact additions), the norm, then the
// indices of the element pairs.
__global__ void __launch_bounds__(256) quant_cb4_kernel(const float *__restrict__ w, int K, float rk, Levels lv,
                                                        uint8_t *__restrict__ codes, uint16_t *__restrict__ norms) {
    __shared__ int fmax_part[256];
    __shared__ Sum320 part[256];
    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    const float *wr = w + n * int64_t(K);
    auto expo = [](uint32_t bits) { return max(int((bits >> 23) & 0xFFu), 1); };
    int fm = 1;
    for (int k = tid; k < K; k += 256) fm = max(fm, expo(__float_as_uint(wr[k])));
    fmax_part[tid] = fm;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if (tid < s) fmax_part[tid] = max(fmax_part[tid], fmax_part[tid + s]);
        __syncthreads();
    }
    const int F = fmax_part[0];
    Sum320 acc = {{0, 0, 0, 0, 0}, 0};
    for (int k = tid; k < K; k += 256) {
        const uint32_t bits = __float_as_uint(wr[k]) & 0x7FFFFFFFu;
        const uint64_t m = (bits & 0x7FFFFFu) | (((bits >> 23) & 0xFFu) ? 0x800000u : 0u);
        add_shifted(acc, m * m, 2 * (expo(bits) - F) + SQ_SHIFT);
    }
    part[tid] = acc;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if (tid < s) {
            Sum320 t = part[tid];
            add320(t, part[tid + s]);
            part[tid] = t;
        }
        __syncthreads();
    }
    const float nrm = bf16_sqrt_of_sum(part[0], 2 * F - 300 - SQ_SHIFT);
    const bool ok = nrm > 0.0f;
    for (int p = tid; p < K / 2; p += 256) {
        const float2 x = *reinterpret_cast<const float2 *>(wr + 2 * p);
        uint32_t idx[2] = {0u, 0u};
        if (ok) {
            const float u[2] = {__fdiv_rn(__fmul_rn(x.x, rk), nrm), __fdiv_rn(__fmul_rn(x.y, rk), nrm)};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                double best = fabs((double)u[h] - (double)lv.c[0]);
#pragma unroll
                for (int j = 1; j < 16; ++j) {
                    const double d = fabs((double)u[h] - (double)lv.c[j]);
                    if (d < best) {                      // strict: a tie keeps the lower index
                        best = d;
                        idx[h] = uint32_t(j);
                    }
                }
            }
        }
        codes[n * int64_t(K / 2) + p] = uint8_t(idx[0] | (idx[1] << 4));
    }
    if (tid == 0) norms[n] = __builtin_bit_cast(uint16_t, (__bf16)nrm);   // exact: nrm has 8 bits
}

}  // namespace

namespace {
template <int PG>
hipError_t launch_group(int fmt, bool zp, dim3 grid, const float *w, int64_t N, int64_t K, void *codes, void *scales,
                        void *zeros, hipStream_t st) {
    const dim3 blk(256);
    if (fmt == FMT_INT4 && zp)
        hipLaunchKernelGGL((quant_group_kernel<FMT_INT4, true, PG>), grid, blk, 0, st, w, int(N), int(K),
                           (uint8_t *)codes, scales, (uint8_t *)zeros);
    else if (fmt == FMT_INT4)
        hipLaunchKernelGGL((quant_group_kernel<FMT_INT4, false, PG>), grid, blk, 0, st, w, int(N), int(K),
                           (uint8_t *)codes, scales, (uint8_t *)zeros);
    else if (fmt == FMT_INT8)
        hipLaunchKernelGGL((quant_group_kernel<FMT_INT8, false, PG>), grid, blk, 0, st, w, int(N), int(K),
                           (uint8_t *)codes, scales, (uint8_t *)zeros);
    else
        hipLaunchKernelGGL((quant_group_kernel<FMT_MXFP4, false, PG>), grid, blk, 0, st, w, int(N), int(K),
                           (uint8_t *)codes, scales, (uint8_t *)zeros);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize(int fmt, int64_t N, int64_t K, int group, bool zp, const float *w,
                           const float *levels_host, void *codes, void *scales, void *zeros, hipStream_t st) {
    if (fmt == FMT_CB4) {
        Levels lv;
        for (int j = 0; j < 16; ++j) lv.c[j] = levels_host[j];
        const float rk = (float)sqrt((double)K);         // float32 of the correctly rounded sqrt
        hipLaunchKernelGGL(quant_cb4_kernel, dim3(unsigned(N)), dim3(256), 0, st, w, int(K), rk, lv, (uint8_t *)codes,
                           (uint16_t *)scales);
        return hipGetLastError();
    }
    const int64_t groups = N * (K / group);
    const int per_block = 4 * (64 / std::min(group / 2, 64));   // groups per 256-thread block
    const dim3 grid(unsigned((groups + per_block - 1) / per_block));
    switch (group) {
        case 32: return launch_group<16>(fmt, zp, grid, w, N, K, codes, scales, zeros, st);
        case 64: return launch_group<32>(fmt, zp, grid, w, N, K, codes, scales, zeros, st);
        case 128: return launch_group<64>(fmt, zp, grid, w, N, K, codes, scales, zeros, st);
        default: return launch_group<128>(fmt, zp, grid, w, N, K, codes, scales, zeros, st);
    }
    return hipGetLastError();
}

}  // namespace ql
