// Device layout of packed weights and the launch plan of the linear kernels.
//
// Device layout (all formats).  The weight [N, K] is cut into tiles of 16 output
// columns by one "chunk" of the input dimension (128 inputs for the 4-bit formats,
// 64 for INT8), 1024 bytes each.  Tiles of one column block are consecutive along K,
// so a wave that owns a column block streams one contiguous run of memory.  Inside a
// tile, lane l (0..63) of a wavefront reads the 16 bytes at l*16 with one dwordx4
// load: column (l mod 16) and, for each 32-wide k-step of the chunk, the 8 inputs
// 8*(l div 16) .. +7 -- exactly the B-operand slice that lane feeds to a
// v_mfma_f32_16x16x32_bf16.  The nibble order inside each 32-bit k-step word is
// chosen per format so that the register decode needs no element shuffles
// (see ql_decode.hpp).  This is the offline shuffle of the Petit package description
// ("Techniques and performance"): all layout work happens once, at pack time.
//
// Scales are stored per column tile as well, [tile][group][16 columns], so each lane
// loads its own column's scale; MXFP4 keeps the four E8M0 codes of one chunk and one
// column in one 32-bit word.  Codebook weights carry float32 row scales.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

namespace ql {

enum : int { FMT_INT4 = 0, FMT_MXFP4 = 1, FMT_INT8 = 2, FMT_CB4 = 3 };

constexpr int TILE_N = 16;
constexpr int TILE_BYTES = 1024;
constexpr int CB_AUX_BYTES = 128;   // codebook record: centroids, bf16 LUT, alpha
constexpr int WG_THREADS = 256;     // four wavefronts per workgroup

__host__ __device__ constexpr int chunk_k(int fmt) { return fmt == FMT_INT8 ? 64 : 128; }

inline size_t round256(size_t v) { return (v + 255) & ~size_t(255); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Layout {
    int fmt = 0, group = 0;
    bool zeros = false;
    int64_t N = 0, K = 0;
    int64_t Np = 0, Kp = 0;     // padded to whole tiles / chunks
    int64_t ntiles = 0;         // Np / 16
    int64_t kchunks = 0;        // Kp / chunk
    int64_t ngroups = 0;        // Kp / group (INT4, INT8)
    size_t w_bytes = 0, s_bytes = 0, aux_bytes = 0;
};

inline Layout make_layout(int fmt, int64_t N, int64_t K, int group, bool zeros) {
    Layout L;
    L.fmt = fmt;
    L.group = group;
    L.zeros = zeros;
    L.N = N;
    L.K = K;
    const int ch = chunk_k(fmt);
    L.Np = ceil_div(N, TILE_N) * TILE_N;
    L.Kp = ceil_div(K, ch) * ch;
    L.ntiles = L.Np / TILE_N;
    L.kchunks = L.Kp / ch;
    L.w_bytes = round256(size_t(L.ntiles) * size_t(L.kchunks) * TILE_BYTES);
    if (fmt == FMT_INT4 || fmt == FMT_INT8) {
        L.ngroups = L.Kp / group;
        L.s_bytes = round256(size_t(L.ntiles) * size_t(L.ngroups) * TILE_N * 2);
        L.aux_bytes = zeros ? round256(size_t(L.ntiles) * size_t(L.ngroups) * (TILE_N / 2)) : 0;
    } else if (fmt == FMT_MXFP4) {
        L.s_bytes = round256(size_t(L.ntiles) * size_t(L.kchunks) * TILE_N * 4);
        L.aux_bytes = 0;
    } else {
        L.s_bytes = round256(size_t(L.Np) * 4 + size_t(L.Np) * 2);
        L.aux_bytes = CB_AUX_BYTES;
    }
    return L;
}

// Schedules of the INT8-compute (W4A8 / W8A8) ring kernel: MT x NT 16x16 tiles per
// wavefront, WM x WN wavefronts.
struct A8Tile {
    int MT, NT, WM, WN;
};
constexpr int NUM_A8_TILES = 5;
constexpr A8Tile A8_TILES[NUM_A8_TILES] = {
    {8, 3, 1, 4}, {4, 4, 2, 2}, {4, 4, 1, 4}, {2, 4, 1, 4}, {1, 4, 1, 4},
};
// the largest tile that still gives every compute unit a workgroup, else the smallest
inline int default_a8_tile(int64_t M, int64_t N, int num_cu) {
    for (int t = 0; t < NUM_A8_TILES; ++t) {
        const A8Tile &c = A8_TILES[t];
        if (ceil_div(M, 16 * c.MT * c.WM) * ceil_div(N, 16 * c.NT * c.WN) >= num_cu) return t;
    }
    return NUM_A8_TILES - 1;
}

// Launch arguments of the linear kernels.
struct GemmArgs {
    const uint16_t *x;     // bf16 activations, row stride ldx elements
    const uint8_t *w;      // packed tiles
    const uint8_t *s;      // packed scales
    const uint8_t *z;      // packed zero-points (INT4 with zeros)
    const uint8_t *aux;    // codebook record (CB4 only, else null)
    const uint16_t *bias;  // bf16 [N] or null
    void *out;             // [M, N] bf16 or float32
    float *ws;             // split-K partial sums [ks][M][Np]
    int M, N, K, ldx, Np;
    int ntiles, kchunks, ngroups;
    int cps, ks;           // chunks per split, number of splits
    int swiglu, out_f32;
    uint32_t w_bytes, s_bytes, z_bytes;
    // grouped (mixture-of-experts) mode, ring tiles only: the grid has `slots` row-block
    // slots; tile_map[2 s] = expert of slot s (-1: unused), tile_map[2 s + 1] = its first
    // row within the expert; expert e owns rows offsets[e] .. offsets[e+1]-1 of x and
    // out, and its packed buffers start e * stride bytes after w, s, z (aux: e * 128)
    const int *tile_map;   // null: dense
    const int *offsets;
    uint64_t w_stride, s_stride, z_stride;
    int slots;
};

// Schedules compiled into the library.
//   kind 0 (decode, M <= 16): one workgroup per 16*NT output columns over the whole
//           input dimension, split over WK wavefronts and reduced in LDS;
//   kind 2 (LDS ring): WM x WN wavefronts, each 16*MT rows x 16*NT columns, times WK
//           wavefronts that share a tile and split each chunk's k-steps (WK = 4 takes
//           the four k-steps of a 4-bit chunk; INT8 chunks have two, so INT8 runs such
//           a tile with WK = 2: the same tile and grid, half the wavefronts); activations
//           and packed weights staged chunk by chunk into a PF-deep LDS ring by direct
//           buffer->LDS loads (ql_gemm_lds.hpp); the input dimension may be split over
//           workgroups (then a reduce kernel adds the partial sums in split order).
// PF = weight chunks in flight per wavefront (kind 0) or ring depth (kind 2).  The
// decode schedules keep two chunks in flight, but for two single-tile ones (four and
// eight chunks, for small chunks over a long input dimension): a plain stream of HBM reads on
// MI355X is fastest with about 8 KiB outstanding per wavefront and slows with more (a
// 58.7 MB read at 16 or 24 KiB per wavefront took 9-25% longer), and the decode rings
// measured the same way (two-deep against three- and four-deep: 3-8% faster at the
// 4096 x 4096 INT4, 4096 x 14336 MXFP4 and 8192 x 28672 INT8 workloads).
// CP (ring schedules with WK = 2): the two wavefronts of a tile take alternate chunks,
// each all of its chunk's k-steps, instead of alternate k-steps of every chunk; a ring
// stage holds two chunks, so each workgroup walks half as many ring steps (and
// barriers) in series.
struct TileCfg { int kind, MT, NT, PF, WK, WM, WN, CP; };
constexpr int NUM_TILE_CFGS = 25;
constexpr TileCfg TILE_CFGS[NUM_TILE_CFGS] = {
    {0, 1, 1, 2, 8, 1, 1, 0}, {0, 1, 2, 2, 8, 1, 1, 0}, {0, 1, 4, 2, 4, 1, 1, 0}, {0, 1, 1, 8, 4, 1, 1, 0},
    {2, 2, 3, 4, 2, 1, 2, 0}, {2, 2, 2, 4, 2, 1, 4, 0}, {2, 4, 3, 4, 2, 1, 2, 0}, {2, 4, 2, 4, 2, 1, 4, 0},
    {2, 8, 3, 3, 1, 1, 4, 0}, {2, 8, 4, 3, 1, 1, 4, 0}, {2, 4, 4, 3, 1, 2, 2, 0}, {2, 4, 3, 4, 1, 1, 4, 0},
    {2, 2, 4, 4, 1, 1, 4, 0}, {2, 8, 3, 3, 2, 1, 4, 0}, {2, 4, 4, 3, 2, 1, 4, 1}, {2, 4, 4, 4, 2, 1, 4, 0},
    {2, 4, 3, 4, 2, 1, 4, 0}, {2, 2, 2, 4, 2, 1, 4, 1}, {2, 4, 3, 5, 1, 1, 4, 0},
    {0, 1, 3, 2, 4, 1, 1, 0}, {0, 1, 7, 2, 4, 1, 1, 0},
    {2, 4, 4, 2, 2, 1, 4, 0}, {2, 2, 3, 4, 4, 1, 2, 0},
    {0, 1, 1, 4, 8, 1, 1, 0}, {0, 1, 1, 2, 4, 1, 1, 0},
};

// Rows / columns of output covered by one workgroup of a tile or LDS-ring schedule.
__host__ __device__ constexpr int cfg_rows(const TileCfg &t) { return 16 * t.MT * (t.kind == 2 ? t.WM : 1); }
__host__ __device__ constexpr int cfg_ntiles(const TileCfg &t) { return t.kind == 0 ? t.NT : t.NT * t.WN; }
// One stage of a decode wavefront's LDS ring: NT packed weight tiles, the chunk's
// scale words and zero-point words (256-byte blocks), then the activation block of 16
// rows x one chunk of bf16; with the fused SwiGLU input stage (sw) the batch's rows fit
// one activation load, so the block is that load's 1 KiB, followed by one more 1 KiB
// block for the gate rows (the up rows go to the activation block, where h replaces
// them).
__host__ __device__ constexpr int gemv_spc(int fmt, int gs) {
    return (fmt == FMT_INT4 || fmt == FMT_INT8) ? (gs <= chunk_k(fmt) / 32 ? chunk_k(fmt) / 32 / gs : 1) : 1;
}
__host__ __device__ constexpr int gemv_scale_blocks(int fmt, int gs, int nt) {
    return (fmt == FMT_INT4 || fmt == FMT_INT8) ? (nt * gemv_spc(fmt, gs) * 8 + 63) / 64
                                               : (fmt == FMT_MXFP4 ? (nt * 16 + 63) / 64 : 0);
}
__host__ __device__ constexpr int gemv_zero_blocks(int fmt, bool zp, int gs, int nt) {
    return (fmt == FMT_INT4 && zp) ? (nt * gemv_spc(fmt, gs) * 2 + 63) / 64 : 0;
}
// activation rows of one 1 KiB load: 64 16-byte pieces, chunk_k(fmt) / 8 pieces a row
__host__ __device__ constexpr int gemv_rows_per_load(int fmt) { return 64 / (chunk_k(fmt) / 8); }
__host__ __device__ constexpr int gemv_stage_bytes(int fmt, bool zp, int gs, int nt, bool sw = false, bool x1 = false) {
    return nt * TILE_BYTES + 256 * (gemv_scale_blocks(fmt, gs, nt) + gemv_zero_blocks(fmt, zp, gs, nt)) +
           (sw ? 2048 : (x1 ? 1024 : 16 * chunk_k(fmt) * 2));
}
constexpr int LDS_BYTES_MAX = 160 * 1024;
// ring depth: PF stages per wavefront, fewer if they would not fit the LDS
__host__ __device__ constexpr int gemv_ring_depth(int fmt, bool zp, int gs, int nt, int wk, int pf, bool sw = false,
                                                 bool x1 = false) {
    return pf * wk * gemv_stage_bytes(fmt, zp, gs, nt, sw, x1) <= LDS_BYTES_MAX
               ? pf
               : LDS_BYTES_MAX / (wk * gemv_stage_bytes(fmt, zp, gs, nt, sw, x1));
}
__host__ __device__ constexpr int gemv_lds_bytes(int fmt, bool zp, int gs, int nt, int wk, int pf, bool sw = false,
                                                bool x1 = false) {
    return wk * gemv_ring_depth(fmt, zp, gs, nt, wk, pf, sw, x1) * gemv_stage_bytes(fmt, zp, gs, nt, sw, x1);
}
// k-parts a ring schedule runs with for a format: its WK where the chunk's k-steps
// divide evenly, else 2
__host__ __device__ constexpr int ring_wk(int fmt, int wk) { return (chunk_k(fmt) / 32) % wk == 0 ? wk : 2; }
// LDS of a ring schedule: PF stages of activations + packed tiles + every wavefront's
// scale and zero-point words, or, when WK > 1, the hand-over of the accumulators of
// the WK - 1 later k-parts if that is larger.
__host__ __device__ constexpr int ring_stage_bytes(int fmt, bool zp, int gs, int wm, int wn, int wk, int mt, int nt) {
    return 16 * mt * wm * chunk_k(fmt) * 2 + nt * wn * TILE_BYTES +
           wm * wn * wk * 256 * (gemv_scale_blocks(fmt, gs, nt) + gemv_zero_blocks(fmt, zp, gs, nt));
}
// ring depth: PF stages of cs chunks, fewer if they would not fit the LDS
__host__ __device__ constexpr int ring_depth(int fmt, bool zp, int gs, int wm, int wn, int wk, int mt, int nt, int pf,
                                             int cs = 1) {
    return pf * cs * ring_stage_bytes(fmt, zp, gs, wm, wn, wk, mt, nt) <= LDS_BYTES_MAX
               ? pf
               : LDS_BYTES_MAX / (cs * ring_stage_bytes(fmt, zp, gs, wm, wn, wk, mt, nt));
}
// pf: the ring depth actually used (ring_depth)
__host__ __device__ constexpr int ring_lds_bytes(int fmt, bool zp, int gs, int wm, int wn, int wk, int mt, int nt,
                                                 int pf, int cs = 1) {
    return pf * cs * ring_stage_bytes(fmt, zp, gs, wm, wn, wk, mt, nt) > (wk - 1) * wm * wn * mt * nt * 1024
               ? pf * cs * ring_stage_bytes(fmt, zp, gs, wm, wn, wk, mt, nt)
               : (wk - 1) * wm * wn * mt * nt * 1024;
}

struct Plan {
    int cfg = 0;          // index into TILE_CFGS
    int mtiles = 1, nblocks = 1, ks = 1, cps = 1;
    bool fuse_swiglu = false;   // the decode kernel forms h from the raw input itself
    bool x1 = false;            // decode: the rows fit one activation load per chunk
    size_t ws_h = 0;            // bytes of the materialised SwiGLU input at offset 0
    size_t ws_bytes = 0;        // ws_h + split-K partial sums
};

// The decode kernel forms the SwiGLU input h itself when M is at most this: every
// workgroup then evaluates silu over the whole input dimension for the batch's rows,
// which costs less than a separate pass over the raw input only while the rows are few.
constexpr int SWIGLU_FUSE_MAX_M = 2;

inline bool is_decode(int cfg) { return TILE_CFGS[cfg].kind == 0; }

// Default schedule by batch size (measured on MI355X, weights read from HBM, over the
// workload shapes and 3072^2 / 8192^2 / 28672 x 4096 / 4096 x 14336 weights):
//   M <= 16      decode kernel, more column tiles per wavefront for wide layers;
//   M <= 32      32 x 128 ring tiles (eight wavefronts, two k-halves; INT4 / INT8 with
//                the k-halves on alternate chunks);
//   M <= 64      64 x 128 ring tiles (eight wavefronts);
//   codebook and MXFP4 weights streamed from HBM (16 MiB and more) with at least 192
//                tiles of 128 x 256: those tiles, one wavefront per 128 x 64 (fewer
//                activation re-reads per weight tile than the 64-row tiles);
//   then         weights that stay in the caches: 32 x 96 tiles up to M = 512 (with four
//                k-parts, eight wavefronts, where those tiles come to between three
//                quarters of and one workgroup per CU: no split, and no second workgroup
//                on a CU to hide the first one's waits); 64 x 256
//                tiles with two k-halves up to M = 1024 but for cache-resident INT8 (INT4
//                and INT8 streamed from HBM: the k-halves on alternate chunks, three
//                stages of two chunks; else a two-deep ring);
//   larger M     128 x 192 ring tiles, two wavefronts per tile (INT4: one wavefront per
//                tile, whose group accumulators need the registers).
// Split-K is added by make_plan when the tiles alone do not fill the machine.
// Decode schedule: the one whose busiest compute unit streams the fewest column tiles,
// counting one resident workgroup per CU (256 CUs), ties to the wider schedule (fewer
// rounds of workgroups).  Candidates in order of columns per workgroup: 1, 2, 3, 4, 7.
// One column tile per workgroup over a long input dimension (each of the eight
// wavefronts walking 12 chunks or more) at up to 4 rows (one activation load per chunk)
// keeps four chunks in flight instead of two, since such a chunk is a small load
// (measured at 4096 x 14336: 8.9 against 9.3 us at M = 1; at M = 16, with four
// activation loads per chunk, and at 4096 x 4096, four chunks per wavefront, two-deep
// is as fast or faster).
// When the rows fit one activation load (the one-load stage: 36 KiB of LDS for the
// single-tile schedule, four workgroups per CU) and there are at least four column tiles
// per CU, one tile per workgroup streams best (measured at 28672 x 4096 MXFP4: 13.15
// against 14.72 us at M = 1; at 8192 x 28672, two tiles per CU, two-tile workgroups stay
// ahead).
inline int decode_cfg(int64_t ntiles, int64_t kchunks, int64_t M, int64_t rows_per_load) {
    constexpr int cands[] = {0, 1, 19, 2, 20};
    int best = 0;
    int64_t best_load = -1;
    for (int c : cands) {
        const int nt = TILE_CFGS[c].NT;
        const int64_t load = ceil_div(ceil_div(ntiles, nt), 256) * nt;
        if (best_load < 0 || load <= best_load) {
            best = c;
            best_load = load;
        }
    }
    if (M <= rows_per_load && ntiles >= 4 * 256) best = 0;
    if (best == 0 && M <= 4 && ceil_div(kchunks, int64_t(TILE_CFGS[0].WK)) >= 12) best = 23;
    return best;
}

inline int default_cfg(const Layout &L, int64_t M) {
    const bool intf = L.fmt == FMT_INT4 || L.fmt == FMT_INT8;
    if (M <= 16) return decode_cfg(L.ntiles, L.kchunks, M, gemv_rows_per_load(L.fmt));
    if (M <= 32) return intf ? 17 : 5;
    if (M <= 64) return 7;
    const bool streamed = L.w_bytes >= (size_t(16) << 20);
    const bool lut4 = L.fmt == FMT_CB4 || L.fmt == FMT_MXFP4;
    if (lut4 && streamed && ceil_div(M, int64_t(128)) * ceil_div(int64_t(L.ntiles), int64_t(16)) >= 192) return 9;
    if (!streamed && M <= 512) {
        const int64_t wgs = ceil_div(M, int64_t(32)) * ceil_div(int64_t(L.ntiles), int64_t(6));
        return (4 * wgs >= 3 * 256 && wgs <= 256) ? 22 : 4;
    }
    if (M <= 1024 && streamed && intf) return 14;
    if (M <= 1024 && (streamed || L.fmt != FMT_INT8)) return 21;
    if (L.fmt == FMT_INT8) return 13;
    return L.fmt == FMT_INT4 ? 8 : 13;
}

// splits <= 0 picks the split count automatically (tile schedules only): enough
// workgroups to give every compute unit one, split-K only when the column blocks alone
// do not, each split holding whole activation blocks and whole groups.
inline Plan make_plan(const Layout &L, int64_t M, int cfg, int splits, int num_cu, bool swiglu) {
    Plan p;
    p.cfg = cfg;
    const TileCfg t = TILE_CFGS[cfg];
    const int ch = chunk_k(L.fmt);
    int64_t span = 1;
    if ((L.fmt == FMT_INT4 || L.fmt == FMT_INT8) && L.group > ch) span = L.group / ch;
    if (t.kind == 0) {
        // decode: the wavefronts of a workgroup split the chunks; cps = chunks per wavefront
        p.mtiles = 1;
        p.nblocks = int(ceil_div(L.ntiles, t.NT));
        int64_t cpw = ceil_div(L.kchunks, t.WK);
        cpw = ceil_div(cpw, span) * span;
        p.cps = int(cpw);
        p.ks = 1;
        p.fuse_swiglu = swiglu && M <= SWIGLU_FUSE_MAX_M;
        p.x1 = !p.fuse_swiglu && M <= gemv_rows_per_load(L.fmt);
        if (swiglu && !p.fuse_swiglu) p.ws_h = round256(size_t(M) * size_t(L.K) * 2);
        p.ws_bytes = p.ws_h;
        return p;
    }
    p.mtiles = int(ceil_div(M, cfg_rows(t)));
    p.nblocks = int(ceil_div(L.ntiles, cfg_ntiles(t)));
    const int64_t wgs = int64_t(p.mtiles) * p.nblocks;
    int64_t ks = splits;
    if (ks <= 0) {
        // enough workgroups to give every compute unit one (a machine already three
        // quarters full is not split: the split costs a reduce pass)
        ks = 4 * wgs < 3 * int64_t(num_cu) ? ceil_div(num_cu, wgs) : 1;
        const int64_t blk = std::max<int64_t>(span, 2);
        ks = std::min<int64_t>(ks, std::max<int64_t>(1, L.kchunks / blk));
    }
    ks = std::max<int64_t>(1, std::min<int64_t>(ks, L.kchunks));
    int64_t cps = ceil_div(L.kchunks, ks);
    cps = ceil_div(cps, span) * span;
    ks = ceil_div(L.kchunks, cps);
    p.ks = int(ks);
    p.cps = int(cps);
    if (swiglu) p.ws_h = round256(size_t(M) * size_t(L.K) * 2);
    p.ws_bytes = p.ws_h + (ks > 1 ? round256(size_t(ks) * size_t(M) * size_t(L.Np) * 4) : 0);
    return p;
}

}  // namespace ql
