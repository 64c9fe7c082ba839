// Register-level decode of one packed k-step (8 inputs of one column) into the eight
// bf16 values a lane feeds to v_mfma_f32_16x16x32_bf16 as its B operand.
//
// The B operand is always an exact bf16 image of the code:
//   INT4   offset-binary code u in 0..15  ->  bf16(128 + u)       (one AND-OR per pair)
//   INT8   offset-binary code u in 0..255 ->  bf16(u - 128) in the tile kernels, bf16(u)
//          in the decode kernel (where one fewer operation per value matters more than
//          the extra activation-sum MFMA)              (byte -> f32 -> bf16)
//   MXFP4  E2M1 code with its E8M0 scale  ->  bf16(e2m1 * 2^(e-127))  (hardware convert)
//   CB4    sign-magnitude index           ->  +-bf16(alpha * c[8 + m])  (byte permutes),
//          and with the two-term operand also +-bf16(alpha * c[8 + m] - that), a second
//          operand for a second MFMA, so the two together carry ~16 bits of the level
// INT4's offset (128, plus 8 or its zero-point), group scales and codebook row scales are
// applied to the float32 accumulators, so no rounding happens before the matrix cores except the
// bf16 rounding of alpha * c (one or two terms) for the codebook.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ql_common.hpp"

namespace ql {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer descriptor word 3 for gfx9-family parts (untyped 32-bit data format).
constexpr int BUF_DWORD3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, BUF_DWORD3);
}

// A descriptor from values the caller knows to be wave-uniform but the compiler may not
// (e.g. derived from loads): taken from the first active lane, so it lives in scalar
// registers and buffer instructions need no per-lane loop.
__device__ inline __amdgpu_buffer_rsrc_t make_uniform_rsrc(const void *base, uint32_t bytes) {
    const uint64_t u = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(u))));
    const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(u >> 32))));
    return make_rsrc(reinterpret_cast<const void *>((hi << 32) | lo), uint32_t(__builtin_amdgcn_readfirstlane(int(bytes))));
}

// Ranged loads: a byte offset at or beyond the descriptor's size reads as zero.
__device__ inline u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ inline uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ inline uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ inline uint32_t ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// Direct buffer -> LDS load of 16 bytes per lane: lane l's bytes land at lds + 16*l
// (lds is wave-uniform).  Counted by vmcnt like any vector-memory load; out-of-range
// offsets write zeros.
__device__ inline void ld128_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
}

// Wait until at most N vector-memory loads of this wavefront are outstanding.  The
// counter is 6 bits wide: a larger N is clamped to 63, which only waits longer.
template <int N0>
__device__ inline void wait_vmcnt() {
    constexpr int N = N0 > 63 ? 63 : N0;
    static_assert(N >= 0, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at bits 15:14; expcnt (6:4)
    // and lgkmcnt (11:8) left at their maxima (no wait)
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct buffer -> LDS load of 4 bytes per lane: lane l's word lands at lds + 4*l.
__device__ inline void ld32_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, off, 0, 0, 0);
}

// wait_vmcnt with a wave-uniform run-time count (a scalar jump over immediates).
__device__ inline void wait_vmcnt_rt(int n) {
#define QL_WAIT_CASE(k) \
    case k: wait_vmcnt<k>(); break;
#define QL_WAIT_CASE8(k) QL_WAIT_CASE(k) QL_WAIT_CASE(k + 1) QL_WAIT_CASE(k + 2) QL_WAIT_CASE(k + 3) \
    QL_WAIT_CASE(k + 4) QL_WAIT_CASE(k + 5) QL_WAIT_CASE(k + 6) QL_WAIT_CASE(k + 7)
    switch (n <= 0 ? 0 : n) {
        QL_WAIT_CASE8(0) QL_WAIT_CASE8(8) QL_WAIT_CASE8(16) QL_WAIT_CASE8(24)
        QL_WAIT_CASE8(32) QL_WAIT_CASE8(40) QL_WAIT_CASE8(48)
        QL_WAIT_CASE(56) QL_WAIT_CASE(57) QL_WAIT_CASE(58) QL_WAIT_CASE(59) QL_WAIT_CASE(60) QL_WAIT_CASE(61)
        QL_WAIT_CASE(62)
        default: wait_vmcnt<63>(); break;
    }
#undef QL_WAIT_CASE8
#undef QL_WAIT_CASE
}

// Activation rows of one chunk in LDS, as loaded by wave-wide direct loads of 1 KiB.
// A row of the chunk (chunk_k(FMT) bf16) is P 16-byte pieces; one load covers RPI whole
// rows, so every load reads full 128-byte lines.  Piece p of row r sits at 16-byte slot
// (r % RPI) * P + (p ^ xswz(r)) of load r / RPI: for any 16 consecutive rows and a fixed
// piece the slots differ in their low 4 bits, so an A-fragment read (16 rows, one piece
// each) is a conflict-free ds_read_b128.
template <int FMT>
struct XBlock {
    static constexpr int P = chunk_k(FMT) * 2 / 16;   // 16 (4-bit formats) or 8 (INT8)
    static constexpr int RPI = 64 / P;                // rows per load
    static constexpr int NI = 16 / RPI;               // loads per 16 rows
    static constexpr int BYTES = NI * 1024;           // bytes per 16 rows
    __host__ __device__ static constexpr int xswz(int r) { return P == 16 ? (r & 15) : ((r >> 1) & 7); }
    // byte offset of (row r, piece p) inside the block
    __host__ __device__ static constexpr int slot(int r, int p) {
        return (r / RPI) * 1024 + ((r % RPI) * P + (p ^ xswz(r))) * 16;
    }
};

// Compiler-only fence: no memory access moves across it (the hardware is not waited).
__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

// Wait until this wavefront's LDS accesses have completed (lgkmcnt(0)), with compiler
// fences on both sides.  A builtin, not assembly text, so that the compiler's own wait
// insertion knows the reads are complete and adds no waits of its own for them later.
__device__ inline void wait_lds() {
    compiler_fence();
    // gfx9 s_waitcnt: lgkmcnt (11:8) = 0; vmcnt (3:0, 15:14) and expcnt (6:4) at maxima
    __builtin_amdgcn_s_waitcnt(0xC07F);
    compiler_fence();
}

__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ inline float f16_bits_to_f32(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// h = bf16(up * silu(gate)) for two packed bf16 pairs, float32 math, one rounding (the
// same function wherever the SwiGLU input stage runs, so every path forms the same h)
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


__device__ inline f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- bit position of element j (0..7) of a k-step inside its 32-bit word -------------
// INT4: pairs (2p, 2p+1) sit at bits 4p and 16+4p, so one shift and one AND-OR give the
// packed bf16 pair.  CB4: the four low nibbles of the bytes hold elements 0,2,1,3 and the
// high nibbles 4,6,5,7, so a byte permute gathers the pairs.  MXFP4: natural order.
__host__ __device__ constexpr int pos_int4(int j) { return 4 * (j >> 1) + 16 * (j & 1); }
__host__ __device__ constexpr int pos_cb4(int j) {
    return 8 * (((j & 1) << 1) | ((j >> 1) & 1)) + 4 * (j >> 2);
}
__host__ __device__ constexpr int pos_mxfp4(int j) { return 4 * j; }

// ---- INT4: bf16 bit pattern 0x4300 | u is exactly 128 + u ------------------------------
__device__ inline u32x4 dec_int4(uint32_t w) {
    const uint32_t m = 0x000F000Fu, e = 0x43004300u;
    u32x4 r;
    r.x = (w & m) | e;
    r.y = ((w >> 4) & m) | e;
    r.z = ((w >> 8) & m) | e;
    r.w = ((w >> 12) & m) | e;
    return r;
}

// ---- INT8: eight offset-binary bytes (two words) -> bf16(u - 128) = bf16(q) (SIGNED: the
// code itself, no activation-sum term needed) or bf16(u) (one operation fewer per value;
// the offset 128 is then folded with the activation sum), both exact ----------------------
template <bool SIGNED>
__device__ inline u32x4 dec_int8(uint32_t d0, uint32_t d1) {
    u32x4 r;
    if constexpr (SIGNED) {
        // flipping bit 7 of every byte turns u into the two's-complement code q; a
        // sign-extending byte select then converts it (one instruction per value)
        const int32_t s0 = int32_t(d0 ^ 0x80808080u), s1 = int32_t(d1 ^ 0x80808080u);
        r.x = pack_bf16x2((float)(int8_t)s0, (float)(int8_t)(s0 >> 8));
        r.y = pack_bf16x2((float)(int8_t)(s0 >> 16), (float)(s0 >> 24));
        r.z = pack_bf16x2((float)(int8_t)s1, (float)(int8_t)(s1 >> 8));
        r.w = pack_bf16x2((float)(int8_t)(s1 >> 16), (float)(s1 >> 24));
    } else {
        r.x = pack_bf16x2((float)(d0 & 0xFFu), (float)((d0 >> 8) & 0xFFu));
        r.y = pack_bf16x2((float)((d0 >> 16) & 0xFFu), (float)(d0 >> 24));
        r.z = pack_bf16x2((float)(d1 & 0xFFu), (float)((d1 >> 8) & 0xFFu));
        r.w = pack_bf16x2((float)((d1 >> 16) & 0xFFu), (float)(d1 >> 24));
    }
    return r;
}

// ---- MXFP4: E8M0 code -> float32 scale 2^(e-127); code 0 is the subnormal 2^-127 and
// code 255 is NaN (a quiet-NaN mantissa bit, set only when e + 1 carries into bit 8) -----
__device__ inline float e8m0_to_f32(uint32_t e) {
    return __uint_as_float(e ? (e << 23) | (((e + 1u) >> 8) << 22) : 0x00400000u);
}
// Codes 1..254 are the float32 exponent field itself: 2^(e-127) has the bits e << 23.
__device__ inline float e8m0_to_f32_normal(uint32_t e) { return __uint_as_float(e << 23); }
// Nonzero when any byte of the word is code 0 or 255, the two codes e << 23 does not give
// (the high bit of a zero byte of w or of ~w survives the borrow test).
__device__ inline uint32_t e8m0_special_bytes(uint32_t w) {
    return (((w - 0x01010101u) & ~w) | ((~w - 0x01010101u) & w)) & 0x80808080u;
}

__device__ inline u32x4 dec_mxfp4(uint32_t w, float scale) {
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    return r;
}

// ---- CB4: magnitude LUT of 8 bf16 values split into low-byte and high-byte planes ------
struct CbLut {
    uint32_t lo0, lo1, hi0, hi1;   // byte m of lo0/lo1 (m < 4 / m >= 4) = low byte of entry m
};

__device__ inline u32x4 dec_cb4(uint32_t w, const CbLut &L) {
    const uint32_t sa = w & 0x07070707u;          // magnitudes of elements 0,2,1,3
    const uint32_t sb = (w >> 4) & 0x07070707u;   // magnitudes of elements 4,6,5,7
    // high bytes with their signs: the sign of the element in byte i of sa is bit 8i+3
    // of w, that of byte i of sb is bit 8i+7; both go to bit 7 of that high byte
    const uint32_t sg = 0x80808080u;
    const uint32_t ha = __builtin_amdgcn_perm(L.hi1, L.hi0, sa) ^ ((w << 4) & sg);
    const uint32_t la = __builtin_amdgcn_perm(L.lo1, L.lo0, sa);
    const uint32_t hb = __builtin_amdgcn_perm(L.hi1, L.hi0, sb) ^ (w & sg);
    const uint32_t lb = __builtin_amdgcn_perm(L.lo1, L.lo0, sb);
    u32x4 r;
    r.x = __builtin_amdgcn_perm(ha, la, 0x06020400u);   // elements 0, 1
    r.y = __builtin_amdgcn_perm(ha, la, 0x07030501u);   // elements 2, 3
    r.z = __builtin_amdgcn_perm(hb, lb, 0x06020400u);   // elements 4, 5
    r.w = __builtin_amdgcn_perm(hb, lb, 0x07030501u);   // elements 6, 7
    return r;
}

// Codebook record (128 bytes) written by the packer:
//   [0, 64)    float32 centroids c[16] as given
//   [64, 80)   CbLut planes of hi_m = bf16(alpha * c[8 + m]), m = 0..7
//   [80, 84)   float32 1/alpha
//   [84, 88)   float32 alpha
//   [88, 104)  CbLut planes of lo_m = bf16(fp32(alpha * c[8 + m]) - hi_m)
//   [104, 108) split: 1 = the kernels use the two-term operand hi + lo
struct CbRecord {
    float centroids[16];
    CbLut lut;
    float inv_alpha;
    float alpha;
    CbLut lut_lo;
    uint32_t split;
    uint32_t pad[5];
};
static_assert(sizeof(CbRecord) == CB_AUX_BYTES, "codebook record size");

// Canonical index j <-> sign-magnitude nibble (bit 3 = sign, bits 0..2 = m) for a
// symmetric codebook (c[15 - j] == -c[j]): j >= 8 is +c[8 + m]; j < 8 is -c[8 + m], m = 7 - j.
__host__ __device__ inline uint32_t cb_index_to_nibble(uint32_t j) { return j >= 8 ? j - 8 : 8u | (7u - j); }
__host__ __device__ inline uint32_t cb_nibble_to_index(uint32_t n) { return (n & 8u) ? 7u - (n & 7u) : 8u + n; }

}  // namespace ql
