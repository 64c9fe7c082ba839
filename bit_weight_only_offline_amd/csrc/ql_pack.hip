// Offline pack / unpack between the canonical weight layout and the device layout, the
// codebook record, and the debug dequantised-tile dump.  One thread per 16-byte lane
// record (weights), per scale element, or per output element (tile dump).
#include <hip/hip_runtime.h>
#include <math.h>

#include "ql_common.hpp"
#include "ql_decode.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

// Canonical 32-bit word (8 nibbles, element j at bits 4j) <-> device k-step word.
template <int FMT, bool SYM>
__device__ inline uint32_t to_device_word(uint32_t cw) {
    uint32_t d = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t nib = (cw >> (4 * j)) & 0xFu;
        if (FMT == FMT_INT4) {
            if (SYM) nib ^= 8u;   // two's complement -> offset binary (q + 8)
            d |= nib << pos_int4(j);
        } else if (FMT == FMT_CB4) {
            d |= cb_index_to_nibble(nib) << pos_cb4(j);
        } else {
            d |= nib << pos_mxfp4(j);
        }
    }
    return d;
}

template <int FMT, bool SYM>
__device__ inline uint32_t to_canonical_word(uint32_t d) {
    uint32_t cw = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t nib;
        if (FMT == FMT_INT4) {
            nib = (d >> pos_int4(j)) & 0xFu;
            if (SYM) nib ^= 8u;
        } else if (FMT == FMT_CB4) {
            nib = cb_nibble_to_index((d >> pos_cb4(j)) & 0xFu);
        } else {
            nib = (d >> pos_mxfp4(j)) & 0xFu;
        }
        cw |= nib << (4 * j);
    }
    return cw;
}

// ---- 4-bit weights ---------------------------------------------------------------------
template <int FMT, bool SYM>
__global__ void __launch_bounds__(256) pack4_kernel(const uint32_t *__restrict__ codes, u32x4 *__restrict__ dst,
                                                    int N, int K, int ntiles, int kchunks) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(ntiles) * kchunks * 64) return;
    const int lane = int(gid & 63);
    const int64_t tile = gid >> 6;
    const int nt = int(tile / kchunks), kc = int(tile % kchunks);
    const int g = lane >> 4, c = lane & 15;
    const int n = nt * TILE_N + c;
    u32x4 out;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k8 = kc * 128 + 32 * t + 8 * g;
        uint32_t cw = 0;
        if (n < N && k8 < K) cw = codes[(int64_t(n) * K + k8) / 8];
        out[t] = to_device_word<FMT, SYM>(cw);
    }
    dst[gid] = out;
}

template <int FMT, bool SYM>
__global__ void __launch_bounds__(256) unpack4_kernel(const u32x4 *__restrict__ src, uint32_t *__restrict__ codes,
                                                      int N, int K, int ntiles, int kchunks) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(ntiles) * kchunks * 64) return;
    const int lane = int(gid & 63);
    const int64_t tile = gid >> 6;
    const int nt = int(tile / kchunks), kc = int(tile % kchunks);
    const int g = lane >> 4, c = lane & 15;
    const int n = nt * TILE_N + c;
    const u32x4 v = src[gid];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k8 = kc * 128 + 32 * t + 8 * g;
        if (n < N && k8 < K) codes[(int64_t(n) * K + k8) / 8] = to_canonical_word<FMT, SYM>(v[t]);
    }
}

// ---- INT8 weights: two k-steps of 8 bytes per lane, stored offset-binary (q ^ 0x80) ---
__global__ void __launch_bounds__(256) pack8_kernel(const u32x2 *__restrict__ codes, u32x4 *__restrict__ dst,
                                                    int N, int K, int ntiles, int kchunks) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(ntiles) * kchunks * 64) return;
    const int lane = int(gid & 63);
    const int64_t tile = gid >> 6;
    const int nt = int(tile / kchunks), kc = int(tile % kchunks);
    const int g = lane >> 4, c = lane & 15;
    const int n = nt * TILE_N + c;
    u32x4 out;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int k8 = kc * 64 + 32 * t + 8 * g;
        u32x2 v = {0u, 0u};
        if (n < N && k8 < K) v = codes[(int64_t(n) * K + k8) / 8];
        out[2 * t] = v.x ^ 0x80808080u;
        out[2 * t + 1] = v.y ^ 0x80808080u;
    }
    dst[gid] = out;
}

__global__ void __launch_bounds__(256) unpack8_kernel(const u32x4 *__restrict__ src, u32x2 *__restrict__ codes,
                                                      int N, int K, int ntiles, int kchunks) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(ntiles) * kchunks * 64) return;
    const int lane = int(gid & 63);
    const int64_t tile = gid >> 6;
    const int nt = int(tile / kchunks), kc = int(tile % kchunks);
    const int g = lane >> 4, c = lane & 15;
    const int n = nt * TILE_N + c;
    const u32x4 v = src[gid];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int k8 = kc * 64 + 32 * t + 8 * g;
        if (n < N && k8 < K) {
            u32x2 o;
            o.x = v[2 * t] ^ 0x80808080u;
            o.y = v[2 * t + 1] ^ 0x80808080u;
            codes[(int64_t(n) * K + k8) / 8] = o;
        }
    }
}

// ---- 16-bit group scales [N, NG] <-> [tile][group][16] --------------------------------
__global__ void __launch_bounds__(256) pack_scale16_kernel(const uint16_t *__restrict__ s, uint16_t *__restrict__ dst,
                                                           int N, int NG, int ntiles, int ngp, int dir) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(ntiles) * ngp * TILE_N) return;
    const int c = int(gid & 15);
    const int64_t r = gid >> 4;
    const int nt = int(r / ngp), grp = int(r % ngp);
    const int n = nt * TILE_N + c;
    const bool ok = n < N && grp < NG;
    if (dir == 0) {
        dst[gid] = ok ? s[int64_t(n) * NG + grp] : uint16_t(0);
    } else if (ok) {
        const_cast<uint16_t *>(s)[int64_t(n) * NG + grp] = dst[gid];
    }
}

// ---- 4-bit zero-points [N, NG] bytes <-> [tile][group][8 bytes] -----------------------
__global__ void __launch_bounds__(256) pack_zeros_kernel(const uint8_t *__restrict__ z, uint8_t *__restrict__ dst,
                                                         int N, int NG, int ntiles, int ngp, int dir) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(ntiles) * ngp * 8) return;
    const int p = int(gid & 7);
    const int64_t r = gid >> 3;
    const int nt = int(r / ngp), grp = int(r % ngp);
    const int n0 = nt * TILE_N + 2 * p;
    if (dir == 0) {
        uint32_t lo = (n0 < N && grp < NG) ? (z[int64_t(n0) * NG + grp] & 0xFu) : 0u;
        uint32_t hi = (n0 + 1 < N && grp < NG) ? (z[int64_t(n0 + 1) * NG + grp] & 0xFu) : 0u;
        dst[gid] = uint8_t(lo | (hi << 4));
    } else {
        const uint8_t b = dst[gid];
        uint8_t *zo = const_cast<uint8_t *>(z);
        if (n0 < N && grp < NG) zo[int64_t(n0) * NG + grp] = b & 0xF;
        if (n0 + 1 < N && grp < NG) zo[int64_t(n0 + 1) * NG + grp] = b >> 4;
    }
}

// ---- MXFP4 scales [N, K/32] bytes <-> [tile][chunk][16] words (4 codes each) ----------
__global__ void __launch_bounds__(256) pack_e8m0_kernel(const uint8_t *__restrict__ s, uint32_t *__restrict__ dst,
                                                        int N, int NB, int ntiles, int kchunks, int dir) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(ntiles) * kchunks * TILE_N) return;
    const int c = int(gid & 15);
    const int64_t r = gid >> 4;
    const int nt = int(r / kchunks), kc = int(r % kchunks);
    const int n = nt * TILE_N + c;
    if (dir == 0) {
        uint32_t word = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int b = kc * 4 + t;
            const uint32_t e = (n < N && b < NB) ? s[int64_t(n) * NB + b] : 127u;
            word |= e << (8 * t);
        }
        dst[gid] = word;
    } else {
        const uint32_t word = dst[gid];
        uint8_t *so = const_cast<uint8_t *>(s);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int b = kc * 4 + t;
            if (n < N && b < NB) so[int64_t(n) * NB + b] = uint8_t(word >> (8 * t));
        }
    }
}

// ---- CB4 row scales: s_n = fp32(norm_n) / fp32(sqrt K); the bf16 norms are kept too ----
__global__ void __launch_bounds__(256) pack_cb_scales_kernel(const uint16_t *__restrict__ norms, float *__restrict__ rs,
                                                             uint16_t *__restrict__ keep, int N, int Np, float sqrt_k) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= Np) return;
    const uint16_t b = n < N ? norms[n] : uint16_t(0);
    keep[n] = b;
    rs[n] = bf16_bits_to_f32(b) / sqrt_k;   // IEEE float32 division
}

__global__ void __launch_bounds__(256) unpack_cb_scales_kernel(const uint16_t *__restrict__ keep,
                                                               uint16_t *__restrict__ norms, int N) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n < N) norms[n] = keep[n];
}

// ---- CB4 record: choose alpha in [1, 2) (steps of 2^-12) minimising the summed squared
// relative bf16 rounding error of alpha * c[8 + m], then store the LUT planes of the
// leading term hi_m = bf16(alpha c[8 + m]) and of the residual lo_m = bf16(alpha c[8 + m]
// - hi_m), and choose between the one-term and the two-term operand.
//
// The one-term operand rounds each level once to bf16 (about 1e-3 relative error after
// alpha).  That error is relative to each row's own output, so a row whose norm stands
// far above the others carries it into outputs that dominate the whole matrix, and the
// error measured against the rms of all outputs grows with max(norm) / rms(norm) (about
// 1.4e-3 at a ratio of one, measured on the 3072 x 3072 workload).  Above a ratio of
// CB_SPLIT_RATIO the kernels take the two-term operand (two MFMAs per fragment, about
// 16 bits per level).  The ratio is a property of the norms alone, decided once here.
struct Centroids { float c[16]; };

constexpr float CB_SPLIT_RATIO = 3.0f;

__device__ inline float bf16_rne(float v) { return __uint_as_float(uint32_t(__builtin_bit_cast(uint16_t, (__bf16)v)) << 16); }

__global__ void __launch_bounds__(256) cb_record_kernel(Centroids cs, const uint16_t *__restrict__ norms, int N,
                                                        CbRecord *__restrict__ rec) {
    __shared__ float best_cost[256];
    __shared__ int best_idx[256];
    __shared__ double sq[256];
    __shared__ float mx[256];
    const int t = threadIdx.x;
    float bc = INFINITY;
    int bi = 0;
    for (int j = 0; j < 16; ++j) {
        const int i = t * 16 + j;
        const float a = 1.0f + float(i) * (1.0f / 4096.0f);
        float cost = 0.0f;
        for (int m = 0; m < 8; ++m) {
            const float p = a * cs.c[8 + m];
            const float d = (bf16_rne(p) - p) / a;
            cost = fmaf(d, d, cost);
        }
        if (cost < bc) { bc = cost; bi = i; }
    }
    best_cost[t] = bc;
    best_idx[t] = bi;
    // norm statistics: max and the float64 sum of squares, thread-strided then a tree
    double s2 = 0.0;
    float m2 = 0.0f;
    for (int n = t; n < N; n += 256) {
        const float v = fabsf(bf16_bits_to_f32(norms[n]));
        s2 += double(v) * double(v);
        m2 = fmaxf(m2, v);
    }
    sq[t] = s2;
    mx[t] = m2;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s) {
            const float oc = best_cost[t + s];
            const int oi = best_idx[t + s];
            if (oc < best_cost[t] || (oc == best_cost[t] && oi < best_idx[t])) {
                best_cost[t] = oc;
                best_idx[t] = oi;
            }
            sq[t] += sq[t + s];
            mx[t] = fmaxf(mx[t], mx[t + s]);
        }
        __syncthreads();
    }
    if (t == 0) {
        const float a = 1.0f + float(best_idx[0]) * (1.0f / 4096.0f);
        CbRecord r;
        for (int j = 0; j < 16; ++j) r.centroids[j] = cs.c[j];
        uint32_t lo[2] = {0, 0}, hi[2] = {0, 0}, rlo[2] = {0, 0}, rhi[2] = {0, 0};
        for (int m = 0; m < 8; ++m) {
            const float p = a * cs.c[8 + m];
            const float h = bf16_rne(p);
            const uint32_t b = __float_as_uint(h) >> 16;
            const uint32_t rb = __float_as_uint(bf16_rne(p - h)) >> 16;   // p - h is exact in float32
            lo[m >> 2] |= (b & 0xFFu) << (8 * (m & 3));
            hi[m >> 2] |= (b >> 8) << (8 * (m & 3));
            rlo[m >> 2] |= (rb & 0xFFu) << (8 * (m & 3));
            rhi[m >> 2] |= (rb >> 8) << (8 * (m & 3));
        }
        r.lut.lo0 = lo[0];
        r.lut.lo1 = lo[1];
        r.lut.hi0 = hi[0];
        r.lut.hi1 = hi[1];
        r.lut_lo.lo0 = rlo[0];
        r.lut_lo.lo1 = rlo[1];
        r.lut_lo.hi0 = rhi[0];
        r.lut_lo.hi1 = rhi[1];
        r.inv_alpha = 1.0f / a;
        r.alpha = a;
        // max > ratio * rms, i.e. max^2 * N > ratio^2 * sum of squares
        const double rms2n = sq[0];
        r.split = (double(mx[0]) * double(mx[0]) * double(N) > double(CB_SPLIT_RATIO) * CB_SPLIT_RATIO * rms2n) ? 1u : 0u;
        for (int j = 0; j < 5; ++j) r.pad[j] = 0;
        *rec = r;
    }
}

__global__ void copy_centroids_kernel(const CbRecord *__restrict__ rec, float *__restrict__ out) {
    const int j = threadIdx.x;
    if (j < 16) out[j] = rec->centroids[j];
}

// ---- debug dump: out[i][j] = D(W)[n0+i][k0+j] (mode 0) or the bf16 operand (mode 1) ---
template <int FMT>
__global__ void __launch_bounds__(256) dequant_tile_kernel(const u32x4 *__restrict__ w, const uint8_t *__restrict__ s,
                                                           const uint8_t *__restrict__ z, const uint8_t *__restrict__ aux,
                                                           int K, int kchunks, int ngroups, int group, int zeros,
                                                           int n0, int k0, int tn, int tk, int mode, float *__restrict__ out) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= int64_t(tn) * tk) return;
    const int i = int(gid / tk), j = int(gid % tk);
    const int n = n0 + i, k = k0 + j;
    constexpr int CH = chunk_k(FMT);
    const int nt = n / TILE_N, c = n % TILE_N;
    const int kc = k / CH, kin = k % CH;
    const int t = kin / 32, g = (kin % 32) / 8, e = k % 8;
    const int lane = g * 16 + c;
    const u32x4 rec = w[(int64_t(nt) * kchunks + kc) * 64 + lane];
    u32x4 op;
    float scale = 1.0f;
    if (FMT == FMT_INT4) {
        op = dec_int4(rec[t]);
    } else if (FMT == FMT_INT8) {
        op = dec_int8<true>(rec[2 * t], rec[2 * t + 1]);
    } else if (FMT == FMT_MXFP4) {
        const uint32_t sw = reinterpret_cast<const uint32_t *>(s)[(int64_t(nt) * kchunks + kc) * TILE_N + c];
        op = dec_mxfp4(rec[t], e8m0_to_f32((sw >> (8 * t)) & 0xFFu));
    } else {
        const CbRecord *cr = reinterpret_cast<const CbRecord *>(aux);
        op = dec_cb4(rec[t], cr->lut);
    }
    const uint32_t bits = (op[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    float v = bf16_bits_to_f32(bits);
    if (FMT == FMT_CB4) {
        // with the two-term operand the image is hi + lo, exact in float32 (lo is below
        // half an ulp of hi's 8 bits and carries 8 bits itself)
        const CbRecord *cr = reinterpret_cast<const CbRecord *>(aux);
        if (cr->split) {
            const u32x4 op2 = dec_cb4(rec[t], cr->lut_lo);
            v += bf16_bits_to_f32((op2[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
    }
    float d;
    if (mode == 1) {
        d = v;
    } else if (FMT == FMT_INT4 || FMT == FMT_INT8) {
        const int grp = k / group;
        const uint16_t sb = reinterpret_cast<const uint16_t *>(s)[(int64_t(nt) * ngroups + grp) * TILE_N + c];
        scale = (FMT == FMT_INT4) ? f16_bits_to_f32(sb) : bf16_bits_to_f32(sb);
        float off;
        if (FMT == FMT_INT8) {
            off = 0.0f;                          // the INT8 operand is the signed code
        } else if (zeros) {
            const uint8_t zb = z[(int64_t(nt) * ngroups + grp) * 8 + (c >> 1)];
            off = 128.0f + float((zb >> (4 * (c & 1))) & 0xF);
        } else {
            off = 136.0f;
        }
        d = (v - off) * scale;   // (v - off) is an exact small integer
    } else if (FMT == FMT_MXFP4) {
        d = v;
    } else {
        const CbRecord *cr = reinterpret_cast<const CbRecord *>(aux);
        const uint32_t nib = (rec[t] >> pos_cb4(e)) & 0xFu;
        const float rs = reinterpret_cast<const float *>(s)[n];
        d = cr->centroids[cb_nibble_to_index(nib)] * rs;
    }
    out[gid] = d;
}

// Zero the bytes [begin, end) of a packed buffer: the padding behind the last record,
// so that a packed buffer is a deterministic function of its canonical input.
__global__ void __launch_bounds__(256) zero_tail_kernel(uint8_t *__restrict__ p, int64_t begin, int64_t end) {
    const int64_t i = begin + int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < end) p[i] = 0;
}

inline unsigned blocks_for(int64_t n) { return unsigned((n + 255) / 256); }

void zero_tail(void *p, int64_t begin, int64_t end, hipStream_t st) {
    if (p && end > begin)
        hipLaunchKernelGGL(zero_tail_kernel, dim3(blocks_for(end - begin)), dim3(256), 0, st, (uint8_t *)p, begin, end);
}

}  // namespace

hipError_t launch_pack(const Layout &L, const void *codes, const void *scales, const void *aux_in,
                       void *pw, void *ps, void *paux, hipStream_t st) {
    const int N = int(L.N), K = int(L.K), nt = int(L.ntiles), kc = int(L.kchunks);
    const int64_t recs = int64_t(nt) * kc * 64;
    zero_tail(pw, recs * 16, int64_t(L.w_bytes), st);
    if (L.fmt == FMT_INT8) {
        hipLaunchKernelGGL(pack8_kernel, dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const u32x2 *)codes, (u32x4 *)pw, N, K, nt, kc);
    } else if (L.fmt == FMT_INT4 && !L.zeros) {
        hipLaunchKernelGGL((pack4_kernel<FMT_INT4, true>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const uint32_t *)codes, (u32x4 *)pw, N, K, nt, kc);
    } else if (L.fmt == FMT_INT4) {
        hipLaunchKernelGGL((pack4_kernel<FMT_INT4, false>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const uint32_t *)codes, (u32x4 *)pw, N, K, nt, kc);
    } else if (L.fmt == FMT_MXFP4) {
        hipLaunchKernelGGL((pack4_kernel<FMT_MXFP4, false>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const uint32_t *)codes, (u32x4 *)pw, N, K, nt, kc);
    } else {
        hipLaunchKernelGGL((pack4_kernel<FMT_CB4, false>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const uint32_t *)codes, (u32x4 *)pw, N, K, nt, kc);
    }
    if (L.fmt == FMT_INT4 || L.fmt == FMT_INT8) {
        const int NG = int(L.K / L.group), ngp = int(L.ngroups);
        hipLaunchKernelGGL(pack_scale16_kernel, dim3(blocks_for(int64_t(nt) * ngp * TILE_N)), dim3(256), 0, st,
                           (const uint16_t *)scales, (uint16_t *)ps, N, NG, nt, ngp, 0);
        zero_tail(ps, int64_t(nt) * ngp * TILE_N * 2, int64_t(L.s_bytes), st);
        if (L.zeros) {
            hipLaunchKernelGGL(pack_zeros_kernel, dim3(blocks_for(int64_t(nt) * ngp * 8)), dim3(256), 0, st,
                               (const uint8_t *)aux_in, (uint8_t *)paux, N, NG, nt, ngp, 0);
            zero_tail(paux, int64_t(nt) * ngp * 8, int64_t(L.aux_bytes), st);
        }
    } else if (L.fmt == FMT_MXFP4) {
        hipLaunchKernelGGL(pack_e8m0_kernel, dim3(blocks_for(int64_t(nt) * kc * TILE_N)), dim3(256), 0, st,
                           (const uint8_t *)scales, (uint32_t *)ps, N, int(L.K / 32), nt, kc, 0);
        zero_tail(ps, int64_t(nt) * kc * TILE_N * 4, int64_t(L.s_bytes), st);
    } else {
        const int Np = int(L.Np);
        zero_tail(ps, int64_t(Np) * 6, int64_t(L.s_bytes), st);
        const float sqrt_k = float(sqrt(double(L.K)));
        hipLaunchKernelGGL(pack_cb_scales_kernel, dim3(blocks_for(Np)), dim3(256), 0, st,
                           (const uint16_t *)scales, (float *)ps, (uint16_t *)((uint8_t *)ps + size_t(Np) * 4), N, Np,
                           sqrt_k);
        Centroids cs;
        for (int j = 0; j < 16; ++j) cs.c[j] = ((const float *)aux_in)[j];
        hipLaunchKernelGGL(cb_record_kernel, dim3(1), dim3(256), 0, st, cs, (const uint16_t *)scales, N,
                           (CbRecord *)paux);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const Layout &L, const void *pw, const void *ps, const void *paux,
                         void *codes, void *scales, void *aux_out, hipStream_t st) {
    const int N = int(L.N), K = int(L.K), nt = int(L.ntiles), kc = int(L.kchunks);
    const int64_t recs = int64_t(nt) * kc * 64;
    if (L.fmt == FMT_INT8) {
        hipLaunchKernelGGL(unpack8_kernel, dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const u32x4 *)pw, (u32x2 *)codes, N, K, nt, kc);
    } else if (L.fmt == FMT_INT4 && !L.zeros) {
        hipLaunchKernelGGL((unpack4_kernel<FMT_INT4, true>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const u32x4 *)pw, (uint32_t *)codes, N, K, nt, kc);
    } else if (L.fmt == FMT_INT4) {
        hipLaunchKernelGGL((unpack4_kernel<FMT_INT4, false>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const u32x4 *)pw, (uint32_t *)codes, N, K, nt, kc);
    } else if (L.fmt == FMT_MXFP4) {
        hipLaunchKernelGGL((unpack4_kernel<FMT_MXFP4, false>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const u32x4 *)pw, (uint32_t *)codes, N, K, nt, kc);
    } else {
        hipLaunchKernelGGL((unpack4_kernel<FMT_CB4, false>), dim3(blocks_for(recs)), dim3(256), 0, st,
                           (const u32x4 *)pw, (uint32_t *)codes, N, K, nt, kc);
    }
    if (L.fmt == FMT_INT4 || L.fmt == FMT_INT8) {
        const int NG = int(L.K / L.group), ngp = int(L.ngroups);
        hipLaunchKernelGGL(pack_scale16_kernel, dim3(blocks_for(int64_t(nt) * ngp * TILE_N)), dim3(256), 0, st,
                           (const uint16_t *)scales, (uint16_t *)ps, N, NG, nt, ngp, 1);
        if (L.zeros)
            hipLaunchKernelGGL(pack_zeros_kernel, dim3(blocks_for(int64_t(nt) * ngp * 8)), dim3(256), 0, st,
                               (const uint8_t *)aux_out, (uint8_t *)paux, N, NG, nt, ngp, 1);
    } else if (L.fmt == FMT_MXFP4) {
        hipLaunchKernelGGL(pack_e8m0_kernel, dim3(blocks_for(int64_t(nt) * kc * TILE_N)), dim3(256), 0, st,
                           (const uint8_t *)scales, (uint32_t *)ps, N, int(L.K / 32), nt, kc, 1);
    } else {
        hipLaunchKernelGGL(unpack_cb_scales_kernel, dim3(blocks_for(N)), dim3(256), 0, st,
                           (const uint16_t *)((const uint8_t *)ps + size_t(L.Np) * 4), (uint16_t *)scales, N);
        hipLaunchKernelGGL(copy_centroids_kernel, dim3(1), dim3(64), 0, st, (const CbRecord *)paux, (float *)aux_out);
    }
    return hipGetLastError();
}

hipError_t launch_dequant_tile(const Layout &L, const void *pw, const void *ps, const void *paux, int64_t n0,
                               int64_t k0, int64_t tn, int64_t tk, int mode, float *out, hipStream_t st) {
    const unsigned nb = blocks_for(tn * tk);
    const int kc = int(L.kchunks), ng = int(L.ngroups);
#define QL_DQ(F)                                                                                               \
    hipLaunchKernelGGL((dequant_tile_kernel<F>), dim3(nb), dim3(256), 0, st, (const u32x4 *)pw, (const uint8_t *)ps, \
                       (const uint8_t *)paux, (const uint8_t *)paux, int(L.K), kc, ng, L.group, int(L.zeros),   \
                       int(n0), int(k0), int(tn), int(tk), mode, out)
    switch (L.fmt) {
        case FMT_INT4: QL_DQ(FMT_INT4); break;
        case FMT_INT8: QL_DQ(FMT_INT8); break;
        case FMT_MXFP4: QL_DQ(FMT_MXFP4); break;
        default: QL_DQ(FMT_CB4); break;
    }
#undef QL_DQ
    return hipGetLastError();
}

}  // namespace ql
