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

// Launch arguments of the linear kernels.
struct GemmArgs {
    const uint16_t *x;     // bf16 activations, row stride ldx elements
    const uint8_t *w;      // packed tiles
    const uint8_t *s;      // packed scales
    const uint8_t *z;      // packed zero-points (INT4 with zeros)
    const uint8_t *aux;    // codebook record (CB4)
    const uint16_t *bias;  // bf16 [N] or null
    void *out;             // [M, N] bf16 or float32
    float *ws;             // split-K partials [ks][M][Np]
    int M, N, K, ldx, Np;
    int ntiles, kchunks, ngroups;
    int cps, ks;           // chunks per split, number of splits
    int swiglu, out_f32;
    uint32_t w_bytes, s_bytes, z_bytes;
};

// Tile shapes compiled for the linear kernel: MT m-tiles of 16 rows and NT column
// tiles of 16 per wavefront, PF chunks of weights in flight per wavefront.
struct TileCfg { int MT, NT, PF; };
constexpr int NUM_TILE_CFGS = 5;
constexpr TileCfg TILE_CFGS[NUM_TILE_CFGS] = {
    {1, 1, 8}, {1, 2, 4}, {2, 2, 4}, {4, 2, 4}, {8, 2, 2},
};

struct Plan {
    int cfg = 0;          // index into TILE_CFGS
    int mtiles = 1, nblocks = 1, ks = 1, cps = 1;
    size_t ws_bytes = 0;
};

// Chosen by M (rows), the column-tile count and the chunk count: enough workgroups to
// cover every compute unit a few times, split-K only when the columns alone do not.
inline Plan make_plan(const Layout &L, int64_t M, int num_cu) {
    Plan p;
    if (M <= 16)
        p.cfg = (L.ntiles >= 512) ? 1 : 0;
    else if (M <= 32)
        p.cfg = 2;
    else if (M <= 64)
        p.cfg = 3;
    else
        p.cfg = 4;
    const TileCfg t = TILE_CFGS[p.cfg];
    p.mtiles = int(ceil_div(M, 16 * t.MT));
    p.nblocks = int(ceil_div(L.ntiles, 4 * t.NT));
    const int64_t wgs = int64_t(p.mtiles) * p.nblocks;
    const int64_t target = 2 * int64_t(num_cu);
    int64_t ks = 1;
    if (wgs < target) ks = ceil_div(target, wgs);
    // a split keeps at least two chunks and whole groups
    int64_t span = 1;
    if ((L.fmt == FMT_INT4 || L.fmt == FMT_INT8) && L.group > chunk_k(L.fmt))
        span = L.group / chunk_k(L.fmt);
    const int64_t max_ks = std::max<int64_t>(1, L.kchunks / std::max<int64_t>(2, span));
    if (ks > max_ks) ks = max_ks;
    int64_t cps = ceil_div(L.kchunks, ks);
    cps = ceil_div(cps, span) * span;
    ks = ceil_div(L.kchunks, cps);
    p.ks = int(ks);
    p.cps = int(cps);
    p.ws_bytes = ks > 1 ? round256(size_t(ks) * size_t(M) * size_t(L.Np) * 4) : 0;
    return p;
}

}  // namespace ql
