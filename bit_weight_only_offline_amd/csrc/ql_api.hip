// C ABI of the library: argument validation, sizes, schedule choice and launches.
// Every check runs before anything is queued, so an error leaves all outputs untouched.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/qlinear.h"
#include "ql_common.hpp"
#include "ql_decode.hpp"
#include "ql_launch.hpp"

namespace ql {

// The schedule is a pure function of the shape: it assumes the 256 compute units of
// the MI355X / MI350X (gfx950), so workspace sizes can be queried without a device.
constexpr int PLAN_CUS = 256;

}  // namespace ql

using namespace ql;

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape / format validation shared by every entry point.
ql_status check_format(ql_format f, int64_t N, int64_t K, int group, int has_zeros) {
    if (f < QL_INT4 || f > QL_CB4) return QL_E_ARG;
    if (has_zeros != 0 && has_zeros != 1) return QL_E_ARG;
    if (has_zeros && f != QL_INT4) return QL_E_ARG;
    if (N <= 0 || K <= 0 || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 30)) return QL_E_SHAPE;
    if (K % 32 != 0) return QL_E_SHAPE;
    if (f == QL_INT4 || f == QL_INT8) {
        if (group != 32 && group != 64 && group != 128 && group != 256) return QL_E_SHAPE;
        if (K % group != 0) return QL_E_SHAPE;
    } else if (f == QL_MXFP4) {
        if (group != 32) return QL_E_SHAPE;
    }
    const Layout L = make_layout(int(f), N, K, f == QL_CB4 ? 0 : group, has_zeros != 0);
    // 32-bit buffer offsets inside the kernels
    if (L.w_bytes >= (size_t(1) << 32) || L.s_bytes >= (size_t(1) << 32)) return QL_E_SHAPE;
    return QL_OK;
}

Layout layout_of(ql_format f, int64_t N, int64_t K, int group, int has_zeros) {
    return make_layout(int(f), N, K, f == QL_CB4 ? 0 : group, has_zeros != 0);
}

ql_status from_hip(hipError_t e) { return e == hipSuccess ? QL_OK : QL_E_HIP; }

}  // namespace

extern "C" {

int qlinear_version(void) { return 0x000100; }

const char *qlinear_error_string(ql_status s) {
    switch (s) {
        case QL_OK: return "ok";
        case QL_E_ARG: return "invalid argument";
        case QL_E_SHAPE: return "unsupported shape or group size";
        case QL_E_ALIGN: return "misaligned pointer";
        case QL_E_UNSUPPORTED: return "unsupported combination";
        case QL_E_WORKSPACE: return "workspace too small";
        case QL_E_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

ql_status qlinear_packed_bytes(ql_format f, int64_t N, int64_t K, int group, int has_zeros, size_t *w_bytes,
                               size_t *s_bytes, size_t *aux_bytes) {
    if (!w_bytes || !s_bytes || !aux_bytes) return QL_E_ARG;
    const ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    const Layout L = layout_of(f, N, K, group, has_zeros);
    *w_bytes = L.w_bytes;
    *s_bytes = L.s_bytes;
    *aux_bytes = L.aux_bytes;
    return QL_OK;
}

ql_status qlinear_pack(ql_format f, int64_t N, int64_t K, int group, const void *codes, const void *scales,
                       const void *aux_in, void *packed_w, void *packed_s, void *packed_aux, void *stream) {
    const int has_zeros = (f == QL_INT4 && aux_in != nullptr) ? 1 : 0;
    ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    if (!codes || !scales || !packed_w || !packed_s) return QL_E_ARG;
    if ((f == QL_CB4) && (!aux_in || !packed_aux)) return QL_E_ARG;
    if (f == QL_INT4 && has_zeros && !packed_aux) return QL_E_ARG;
    if ((f == QL_INT8 || f == QL_MXFP4) && aux_in) return QL_E_ARG;
    if (!aligned(codes, f == QL_INT8 ? 8 : 4)) return QL_E_ALIGN;
    if (!aligned(scales, f == QL_MXFP4 ? 1 : 2)) return QL_E_ALIGN;
    if (!aligned(packed_w, 16) || !aligned(packed_s, 16) || (packed_aux && !aligned(packed_aux, 16))) return QL_E_ALIGN;
    if (f == QL_CB4) {
        const float *c = static_cast<const float *>(aux_in);
        for (int j = 0; j < 16; ++j) {
            if (!isfinite(c[j])) return QL_E_UNSUPPORTED;
            if (c[15 - j] != -c[j]) return QL_E_UNSUPPORTED;   // sign-magnitude decode needs symmetry
        }
    }
    const Layout L = layout_of(f, N, K, group, has_zeros);
    return from_hip(launch_pack(L, codes, scales, aux_in, packed_w, packed_s, packed_aux, (hipStream_t)stream));
}

ql_status qlinear_quantize(ql_format f, int64_t N, int64_t K, int group, const float *w, const float *levels,
                           void *codes, void *scales, void *zeros, void *stream) {
    const int has_zeros = (f == QL_INT4 && zeros != nullptr) ? 1 : 0;
    ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    if (!w || !codes || !scales) return QL_E_ARG;
    if (f == QL_CB4 ? (levels == nullptr || group != 0) : (levels != nullptr)) return QL_E_ARG;
    if (f != QL_INT4 && zeros) return QL_E_ARG;
    if (!aligned(w, 8) || !aligned(codes, 2) || !aligned(scales, f == QL_MXFP4 ? 1 : 2)) return QL_E_ALIGN;
    if (f == QL_CB4)
        for (int j = 0; j < 16; ++j)
            if (!isfinite(levels[j])) return QL_E_UNSUPPORTED;
    if (f != QL_CB4 && N * (K / group) >= (int64_t(1) << 33)) return QL_E_SHAPE;   // grid of groups / 4
    return from_hip(launch_quantize(int(f), N, K, f == QL_CB4 ? 0 : group, has_zeros != 0, w, levels, codes, scales,
                                    zeros, (hipStream_t)stream));
}

ql_status qlinear_int8_addmm(int64_t N, int64_t K, int group, void *packed_w, void *packed_s, const void *mat1,
                             const void *mat2, int64_t rank, float alpha, float beta, int stochastic, uint64_t seed,
                             void *stream) {
    ql_status st = check_format(QL_INT8, N, K, group, 0);
    if (st != QL_OK) return st;
    if (!packed_w || !packed_s) return QL_E_ARG;
    if (rank < 0 || rank > 256) return QL_E_ARG;
    if (rank > 0 && (!mat1 || !mat2)) return QL_E_ARG;
    if (stochastic != 0 && stochastic != 1) return QL_E_ARG;
    if (!isfinite(alpha) || !isfinite(beta)) return QL_E_ARG;
    if (!aligned(packed_w, 16) || !aligned(packed_s, 16)) return QL_E_ALIGN;
    if (rank > 0 && (!aligned(mat1, 2) || !aligned(mat2, 2))) return QL_E_ALIGN;
    const Layout L = layout_of(QL_INT8, N, K, group, 0);
    return from_hip(launch_lora_merge8(L, packed_w, packed_s, mat1, mat2, int(rank), alpha, beta, stochastic, seed,
                                       (hipStream_t)stream));
}

ql_status qlinear_quantize_activations(const void *x, int64_t M, int64_t K, void *codes, float *scales,
                                        void *stream) {
    if (M < 0 || M >= (int64_t(1) << 31) || K <= 0 || K % 32 != 0 || K >= (int64_t(1) << 30)) return QL_E_SHAPE;
    if (M == 0) return QL_OK;
    if (!x || !codes || !scales) return QL_E_ARG;
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4)) return QL_E_ALIGN;
    return from_hip(launch_quant_act(static_cast<const uint16_t *>(x), int(M), int(K), int(K), 0,
                                     static_cast<int8_t *>(codes), scales, (hipStream_t)stream));
}

ql_status qlinear_a8_workspace_bytes(ql_format f, int64_t M, int64_t N, int64_t K, int group, size_t *bytes) {
    if (!bytes) return QL_E_ARG;
    if (f != QL_INT4 && f != QL_INT8) return QL_E_UNSUPPORTED;
    ql_status st = check_format(f, N, K, group, 0);
    if (st != QL_OK) return st;
    if (group < 64) return QL_E_UNSUPPORTED;
    if (M < 0 || M >= (int64_t(1) << 31)) return QL_E_SHAPE;
    const Layout L = layout_of(f, N, K, group, 0);
    *bytes = M == 0 ? 0 : round256(size_t(M) * size_t(L.Kp)) + round256(size_t(M) * 4);
    return QL_OK;
}

int qlinear_a8_num_tiles(void) { return NUM_A8_TILES; }

ql_status qlinear_a8_tile_shape(int tile, int *rows, int *cols) {
    if (tile < 0 || tile >= NUM_A8_TILES || !rows || !cols) return QL_E_ARG;
    *rows = 16 * A8_TILES[tile].MT * A8_TILES[tile].WM;
    *cols = 16 * A8_TILES[tile].NT * A8_TILES[tile].WN;
    return QL_OK;
}

ql_status qlinear_forward_a8(const void *x, int64_t M, int64_t N, int64_t K, const void *packed_w,
                             const void *packed_s, ql_format f, int group, const void *bias, void *out,
                             ql_dtype out_dtype, void *workspace, size_t workspace_bytes, int tile, void *stream) {
    size_t need = 0;
    ql_status st = qlinear_a8_workspace_bytes(f, M, N, K, group, &need);
    if (st != QL_OK) return st;
    if (out_dtype != QL_BF16 && out_dtype != QL_F32) return QL_E_ARG;
    if (tile < -1 || tile >= NUM_A8_TILES) return QL_E_ARG;
    const Layout L = layout_of(f, N, K, group, 0);
    // the quantised rows are addressed with 32-bit buffer offsets whose bit 31 marks
    // "out of range"
    if (M * L.Kp >= (int64_t(1) << 30) || M * N >= (int64_t(1) << 31)) return QL_E_SHAPE;
    if (M == 0) return QL_OK;
    if (!x || !packed_w || !packed_s || !out) return QL_E_ARG;
    if (!aligned(x, 16) || !aligned(packed_w, 16) || !aligned(packed_s, 16)) return QL_E_ALIGN;
    if (bias && !aligned(bias, 2)) return QL_E_ALIGN;
    if (!aligned(out, out_dtype == QL_F32 ? 4 : 2)) return QL_E_ALIGN;
    if (!workspace || workspace_bytes < need) return QL_E_WORKSPACE;
    if (!aligned(workspace, 256)) return QL_E_ALIGN;
    int8_t *xq = static_cast<int8_t *>(workspace);
    float *xs = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + round256(size_t(M) * size_t(L.Kp)));
    return from_hip(launch_gemm_a8(L, tile < 0 ? default_a8_tile(M, N, PLAN_CUS) : tile, static_cast<const uint16_t *>(x), int(M),
                                   packed_w, packed_s, bias, out, out_dtype == QL_F32, xq, xs, (hipStream_t)stream));
}

ql_status qlinear_unpack(ql_format f, int64_t N, int64_t K, int group, int has_zeros, const void *packed_w,
                         const void *packed_s, const void *packed_aux, void *codes, void *scales, void *aux_out,
                         void *stream) {
    ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    if (!codes || !scales || !packed_w || !packed_s) return QL_E_ARG;
    const bool needs_aux = (f == QL_CB4) || (f == QL_INT4 && has_zeros);
    if (needs_aux && (!packed_aux || !aux_out)) return QL_E_ARG;
    if (!aligned(codes, f == QL_INT8 ? 8 : 4)) return QL_E_ALIGN;
    if (!aligned(scales, f == QL_MXFP4 ? 1 : 2)) return QL_E_ALIGN;
    if (!aligned(packed_w, 16) || !aligned(packed_s, 16) || (packed_aux && !aligned(packed_aux, 16))) return QL_E_ALIGN;
    if (f == QL_CB4 && !aligned(aux_out, 4)) return QL_E_ALIGN;
    const Layout L = layout_of(f, N, K, group, has_zeros);
    return from_hip(launch_unpack(L, packed_w, packed_s, packed_aux, codes, scales, aux_out, (hipStream_t)stream));
}

ql_status qlinear_dequant_tile(ql_format f, int64_t N, int64_t K, int group, int has_zeros, const void *packed_w,
                               const void *packed_s, const void *packed_aux, int64_t n0, int64_t k0, int64_t tn,
                               int64_t tk, int mode, float *out, void *stream) {
    ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    if (!packed_w || !packed_s || !out) return QL_E_ARG;
    if (((f == QL_CB4) || (f == QL_INT4 && has_zeros)) && !packed_aux) return QL_E_ARG;
    if (mode != 0 && mode != 1) return QL_E_ARG;
    if (n0 < 0 || k0 < 0 || tn < 0 || tk < 0 || n0 + tn > N || k0 + tk > K) return QL_E_SHAPE;
    if (tn * tk >= (int64_t(1) << 31)) return QL_E_SHAPE;
    if (!aligned(packed_w, 16) || !aligned(packed_s, 16) || !aligned(out, 4)) return QL_E_ALIGN;
    if (tn == 0 || tk == 0) return QL_OK;
    const Layout L = layout_of(f, N, K, group, has_zeros);
    return from_hip(launch_dequant_tile(L, packed_w, packed_s, packed_aux, n0, k0, tn, tk, mode, out,
                                        (hipStream_t)stream));
}

int qlinear_num_tiles(void) { return NUM_TILE_CFGS; }

ql_status qlinear_tile_shape(int tile, int *rows, int *cols, int *kblock) {
    if (tile < 0 || tile >= NUM_TILE_CFGS || !rows || !cols || !kblock) return QL_E_ARG;
    const TileCfg &t = TILE_CFGS[tile];
    *rows = cfg_rows(t);
    *cols = 16 * cfg_ntiles(t);
    *kblock = t.kind == 0 ? 0 : chunk_k(FMT_INT4);   // 0: no activation staging (decode)
    return QL_OK;
}

}  // extern "C"

namespace {

// Launch-grid limits of the device: the x dimension takes up to 2^31 - 1 workgroups, the
// y and z dimensions 65536 (hipDeviceProp_t::maxGridSize on gfx950); 65535 is used.
constexpr int64_t GRID_X_MAX = (int64_t(1) << 31) - 1;
constexpr int64_t GRID_YZ_MAX = 65535;

// Resolve a (possibly partial) schedule into a launch plan.
ql_status plan_for(ql_format f, int64_t M, int64_t N, int64_t K, int group, int has_zeros, ql_act act,
                   const ql_schedule *sched, Layout *L, Plan *p) {
    *L = layout_of(f, N, K, group, has_zeros);
    int cfg = default_cfg(*L, M);
    int splits = 0;
    if (sched) {
        if (sched->tile >= NUM_TILE_CFGS || sched->tile < -1) return QL_E_ARG;
        if (sched->tile >= 0) cfg = sched->tile;
        splits = sched->splits;
        if (splits < 0) return QL_E_ARG;
    }
    if (is_decode(cfg) && (M > 16 || splits > 1)) return QL_E_UNSUPPORTED;   // decode: M <= 16, no split
    *p = make_plan(*L, M, cfg, splits, PLAN_CUS, act == QL_ACT_SWIGLU);
    // grid: decode (column blocks); ring tiles (row x column blocks, splits)
    const int kind = TILE_CFGS[cfg].kind;
    const int64_t gx = kind == 2 ? int64_t(p->mtiles) * p->nblocks : int64_t(p->nblocks);
    if (gx > GRID_X_MAX || p->ks > GRID_YZ_MAX) return QL_E_UNSUPPORTED;
    return QL_OK;
}

// Grouped (mixture-of-experts) launch: the decode kernel (slots of 16 rows) or ring tiles,
// chosen by the mean number of tokens per expert, one row-block slot per possible tile
// (sum over experts of ceil(T_e / rows) is at most ceil(T / rows) + E), no split of the
// input dimension across workgroups.  Workspace: the expert
// offsets [E + 1] and the slot map [slots][2], both int32.
struct GroupedPlan {
    Plan plan;
    int rows = 0;
    size_t ws_bytes = 0;
    bool fits = true;    // the launch grid is within the device's limits
};
GroupedPlan grouped_plan(int64_t T, int64_t E, int64_t N, int64_t K, ql_format f, int group) {
    GroupedPlan g;
    const Layout L = layout_of(f, N, K, group, 0);
    const int64_t per = (T + E - 1) / E;
    int cfg;
    // (the decode kernel takes the slots as the grid's y dimension: past its limit the
    // 32-row ring tile, with the slots along x, serves instead).  The slots of one column
    // block run in rounds, one expert's weight per round; for experts of one column tile
    // per workgroup the four-wavefront schedule (44 KiB of LDS at 16 rows, three
    // workgroups per CU) overlaps the rounds' ramps and drains (measured: eight
    // 4096 x 14336 MXFP4 experts at 16 tokens, 56.6-60.4 against 62.9-64.4 us with the
    // eight-wavefront one)
    if (per <= 16 && ceil_div(T, 16) + E <= GRID_YZ_MAX) {   // decode, 16-row slots
        cfg = default_cfg(L, 16);
        if (cfg == 0) cfg = 24;
    }
    else if (per <= 48) cfg = (f == QL_INT4 || f == QL_INT8) ? 17 : 5;   // 32 x 128, two waves per tile
    else if (per <= 96) cfg = 16;                        // 64 x 192, two waves per tile
    else cfg = (f == QL_INT4 || f == QL_INT8) ? 8 : 13;  // 128 x 192
    g.plan = make_plan(L, 16, cfg, 1, PLAN_CUS, false);  // column blocks, chunks per wave
    g.rows = is_decode(cfg) ? 16 : cfg_rows(TILE_CFGS[cfg]);
    g.plan.mtiles = int(ceil_div(T, g.rows) + E);
    g.plan.ks = 1;
    if (!is_decode(cfg)) g.plan.cps = int(L.kchunks);
    g.ws_bytes = round256(size_t(E + 1) * 4) + round256(size_t(g.plan.mtiles) * 8);
    g.fits = is_decode(cfg) ? (g.plan.mtiles <= GRID_YZ_MAX)
                            : (int64_t(g.plan.mtiles) * g.plan.nblocks <= GRID_X_MAX);
    return g;
}

}  // namespace

extern "C" {

ql_status qlinear_default_schedule(ql_format f, int64_t M, int64_t N, int64_t K, int group, ql_act act,
                                   ql_schedule *out) {
    if (!out) return QL_E_ARG;
    if (act != QL_ACT_NONE && act != QL_ACT_SWIGLU) return QL_E_ARG;
    if (M <= 0 || M >= (int64_t(1) << 31)) return QL_E_SHAPE;
    ql_status st = check_format(f, N, K, group, 0);
    if (st != QL_OK) return st;
    Layout L;
    Plan p;
    st = plan_for(f, M, N, K, group, 0, act, nullptr, &L, &p);
    if (st != QL_OK) return st;
    out->tile = p.cfg;
    out->splits = p.ks;
    return QL_OK;
}

ql_status qlinear_workspace_bytes_ex(ql_format f, int64_t M, int64_t N, int64_t K, int group, ql_act act,
                                     const ql_schedule *sched, size_t *bytes) {
    if (!bytes) return QL_E_ARG;
    if (act != QL_ACT_NONE && act != QL_ACT_SWIGLU) return QL_E_ARG;
    if (M < 0 || M >= (int64_t(1) << 31)) return QL_E_SHAPE;
    ql_status st = check_format(f, N, K, group, 0);
    if (st != QL_OK) return st;
    if (M == 0) {
        *bytes = 0;
        return QL_OK;
    }
    Layout L;
    Plan p;
    st = plan_for(f, M, N, K, group, 0, act, sched, &L, &p);
    if (st != QL_OK) return st;
    *bytes = p.ws_bytes;
    return QL_OK;
}

ql_status qlinear_workspace_bytes(ql_format f, int64_t M, int64_t N, int64_t K, int group, ql_act act,
                                  size_t *bytes) {
    return qlinear_workspace_bytes_ex(f, M, N, K, group, act, nullptr, bytes);
}

ql_status qlinear_forward_ex(const void *x, int64_t M, int64_t N, int64_t K, const void *packed_w,
                             const void *packed_s, const void *packed_aux, ql_format f, int group, int has_zeros,
                             const void *bias, ql_act act, void *out, ql_dtype out_dtype, void *workspace,
                             size_t workspace_bytes, const ql_schedule *sched, void *stream) {
    ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    if (act != QL_ACT_NONE && act != QL_ACT_SWIGLU) return QL_E_ARG;
    if (out_dtype != QL_BF16 && out_dtype != QL_F32) return QL_E_ARG;
    if (M < 0 || M >= (int64_t(1) << 31)) return QL_E_SHAPE;
    const int64_t ldx = act == QL_ACT_SWIGLU ? 2 * K : K;
    // activations are addressed with 32-bit buffer offsets whose bit 31 marks "out of range"
    if (M * ldx >= (int64_t(1) << 30) || M * N >= (int64_t(1) << 31)) return QL_E_SHAPE;
    if (M == 0) return QL_OK;
    if (!x || !packed_w || !packed_s || !out) return QL_E_ARG;
    if (((f == QL_CB4) || (f == QL_INT4 && has_zeros)) && !packed_aux) return QL_E_ARG;
    if (!aligned(x, 16) || !aligned(packed_w, 16) || !aligned(packed_s, 16)) return QL_E_ALIGN;
    if (packed_aux && !aligned(packed_aux, 16)) return QL_E_ALIGN;
    if (bias && !aligned(bias, 2)) return QL_E_ALIGN;
    if (!aligned(out, out_dtype == QL_F32 ? 4 : 2)) return QL_E_ALIGN;
    Layout L;
    Plan p;
    st = plan_for(f, M, N, K, group, has_zeros, act, sched, &L, &p);
    if (st != QL_OK) return st;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes) return QL_E_WORKSPACE;
        if (!aligned(workspace, 256)) return QL_E_ALIGN;
    }
    const bool decode = is_decode(p.cfg);
    GemmArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint8_t *>(packed_w);
    a.s = static_cast<const uint8_t *>(packed_s);
    a.z = (f == QL_INT4 && has_zeros) ? static_cast<const uint8_t *>(packed_aux) : nullptr;
    a.aux = (f == QL_CB4) ? static_cast<const uint8_t *>(packed_aux) : nullptr;
    a.bias = static_cast<const uint16_t *>(bias);
    a.out = out;
    a.ws = (!decode && p.ks > 1) ? reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + p.ws_h) : nullptr;
    a.M = int(M);
    a.N = int(N);
    a.K = int(K);
    a.ldx = int(ldx);
    a.Np = int(L.Np);
    a.ntiles = int(L.ntiles);
    a.kchunks = int(L.kchunks);
    a.ngroups = int(L.ngroups);
    a.cps = p.cps;
    a.ks = p.ks;
    a.swiglu = (act == QL_ACT_SWIGLU && p.fuse_swiglu) ? 1 : 0;   // the kernel forms h itself
    a.out_f32 = out_dtype == QL_F32 ? 1 : 0;
    a.w_bytes = uint32_t(L.w_bytes);
    a.s_bytes = uint32_t(L.s_bytes);
    a.z_bytes = uint32_t(L.aux_bytes);
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (act == QL_ACT_SWIGLU && !p.fuse_swiglu) {
        // materialise h = bf16(up * silu(gate)) once, at the head of the workspace
        uint16_t *h = static_cast<uint16_t *>(workspace);
        e = launch_swiglu(a.x, h, a.M, a.K, s);
        if (e != hipSuccess) return QL_E_HIP;
        a.x = h;
        a.ldx = a.K;
        a.swiglu = 0;
    }
    switch (f) {
        case QL_INT4: e = launch_gemm_int4(L, p, a, s); break;
        case QL_INT8: e = launch_gemm_int8(L, p, a, s); break;
        case QL_MXFP4: e = launch_gemm_mxfp4(L, p, a, s); break;
        default: e = launch_gemm_cb4(L, p, a, s); break;
    }
    if (e != hipSuccess) return QL_E_HIP;
    if (!decode && p.ks > 1) e = launch_reduce(a, s);
    return from_hip(e);
}

ql_status qlinear_forward(const void *x, int64_t M, int64_t N, int64_t K, const void *packed_w, const void *packed_s,
                          const void *packed_aux, ql_format f, int group, int has_zeros, const void *bias, ql_act act,
                          void *out, ql_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return qlinear_forward_ex(x, M, N, K, packed_w, packed_s, packed_aux, f, group, has_zeros, bias, act, out,
                              out_dtype, workspace, workspace_bytes, nullptr, stream);
}

ql_status qlinear_grouped_workspace_bytes(ql_format f, int64_t T, int64_t E, int64_t N, int64_t K, int group,
                                          size_t *bytes) {
    if (!bytes) return QL_E_ARG;
    ql_status st = check_format(f, N, K, group, 0);
    if (st != QL_OK) return st;
    if (T < 0 || E < 0 || T >= (int64_t(1) << 31) || E >= (int64_t(1) << 20)) return QL_E_SHAPE;
    if (T == 0 || E == 0) {
        *bytes = 0;
        return QL_OK;
    }
    const GroupedPlan gp = grouped_plan(T, E, N, K, f, group);
    if (!gp.fits) return QL_E_SHAPE;
    *bytes = gp.ws_bytes;
    return QL_OK;
}

ql_status qlinear_grouped_forward(const void *x, int64_t T, const int32_t *tokens_per_expert, int64_t E, int64_t N,
                                  int64_t K, const void *packed_w, const void *packed_s, const void *packed_aux,
                                  ql_format f, int group, int has_zeros, const void *bias, void *out,
                                  ql_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    if (out_dtype != QL_BF16 && out_dtype != QL_F32) return QL_E_ARG;
    if (T < 0 || E < 0 || T >= (int64_t(1) << 31) || E >= (int64_t(1) << 20)) return QL_E_SHAPE;
    if (T * K >= (int64_t(1) << 30) || T * N >= (int64_t(1) << 31)) return QL_E_SHAPE;
    if (T == 0 || E == 0) return QL_OK;
    if (!x || !tokens_per_expert || !packed_w || !packed_s || !out) return QL_E_ARG;
    if (((f == QL_CB4) || (f == QL_INT4 && has_zeros)) && !packed_aux) return QL_E_ARG;
    if (!aligned(x, 16) || !aligned(packed_w, 16) || !aligned(packed_s, 16)) return QL_E_ALIGN;
    if (packed_aux && !aligned(packed_aux, 16)) return QL_E_ALIGN;
    if (!aligned(tokens_per_expert, 4) || (bias && !aligned(bias, 2))) return QL_E_ALIGN;
    if (!aligned(out, out_dtype == QL_F32 ? 4 : 2)) return QL_E_ALIGN;
    const Layout L = layout_of(f, N, K, group, has_zeros);
    const GroupedPlan gp = grouped_plan(T, E, N, K, f, group);
    if (!gp.fits) return QL_E_SHAPE;
    if (!workspace || workspace_bytes < gp.ws_bytes) return QL_E_WORKSPACE;
    if (!aligned(workspace, 256)) return QL_E_ALIGN;
    int *offsets = static_cast<int *>(workspace);
    int *tile_map = offsets + round256(size_t(E + 1) * 4) / 4;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_moe_plan(tokens_per_expert, int(E), int(T), gp.rows, gp.plan.mtiles, offsets, tile_map, s);
    if (e != hipSuccess) return QL_E_HIP;
    GemmArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint8_t *>(packed_w);
    a.s = static_cast<const uint8_t *>(packed_s);
    a.z = (f == QL_INT4 && has_zeros) ? static_cast<const uint8_t *>(packed_aux) : nullptr;
    a.aux = (f == QL_CB4) ? static_cast<const uint8_t *>(packed_aux) : nullptr;
    a.bias = static_cast<const uint16_t *>(bias);
    a.out = out;
    a.ws = nullptr;
    a.M = int(T);
    a.N = int(N);
    a.K = int(K);
    a.ldx = int(K);
    a.Np = int(L.Np);
    a.ntiles = int(L.ntiles);
    a.kchunks = int(L.kchunks);
    a.ngroups = int(L.ngroups);
    a.cps = gp.plan.cps;
    a.ks = 1;
    a.swiglu = 0;
    a.out_f32 = out_dtype == QL_F32 ? 1 : 0;
    a.w_bytes = uint32_t(L.w_bytes);
    a.s_bytes = uint32_t(L.s_bytes);
    a.z_bytes = uint32_t(L.aux_bytes);
    a.tile_map = tile_map;
    a.offsets = offsets;
    a.w_stride = L.w_bytes;
    a.s_stride = L.s_bytes;
    a.z_stride = L.aux_bytes;
    a.slots = gp.plan.mtiles;
    switch (f) {
        case QL_INT4: e = launch_gemm_int4(L, gp.plan, a, s); break;
        case QL_INT8: e = launch_gemm_int8(L, gp.plan, a, s); break;
        case QL_MXFP4: e = launch_gemm_mxfp4(L, gp.plan, a, s); break;
        default: e = launch_gemm_cb4(L, gp.plan, a, s); break;
    }
    return from_hip(e);
}

}  // extern "C"

// ---- allocation-free forward ---------------------------------------------------------
// Scratch of qlinear_forward_noalloc: a file-scope device array in place of the caller's
// workspace (split-K partial sums, the materialised SwiGLU input).  Every GPU the library
// runs on holds its own copy, from module load until the process ends.  Host code never
// uses the array's name as an address: the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
namespace {

constexpr size_t SCRATCH_BYTES = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 256;
std::mutex scratch_mu;
void *scratch_dev[SCRATCH_MAX_DEVICES] = {};

// This device's copy of `scratch`, or null when the device cannot be determined, the
// stream belongs to another device than the current one, or the lookup fails.
void *device_scratch(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return nullptr;
    if (stream) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(stream, &sd) != hipSuccess || int(sd) != dev) return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_dev[dev] = p;
    }
    return scratch_dev[dev];
}

}  // namespace

extern "C" {

size_t qlinear_noalloc_scratch_bytes(void) { return SCRATCH_BYTES; }

ql_status qlinear_forward_noalloc(const void *x, int64_t M, int64_t N, int64_t K, const void *packed_w,
                                  const void *packed_s, const void *packed_aux, ql_format f, int group,
                                  int has_zeros, const void *bias, ql_act act, void *out, ql_dtype out_dtype,
                                  void *stream) {
    size_t need = 0;
    ql_status st = check_format(f, N, K, group, has_zeros);
    if (st != QL_OK) return st;
    if (act != QL_ACT_NONE && act != QL_ACT_SWIGLU) return QL_E_ARG;
    if (M < 0 || M >= (int64_t(1) << 31)) return QL_E_SHAPE;
    if (M > 0) {
        Layout L;
        Plan p;
        st = plan_for(f, M, N, K, group, has_zeros, act, nullptr, &L, &p);
        if (st != QL_OK) return st;
        need = p.ws_bytes;
    }
    if (need > SCRATCH_BYTES) return QL_E_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        ws = device_scratch((hipStream_t)stream);
        if (!ws) return QL_E_HIP;
    }
    // the same validation and kernels as qlinear_forward(), with the scratch as workspace
    return qlinear_forward_ex(x, M, N, K, packed_w, packed_s, packed_aux, f, group, has_zeros, bias, act, out,
                              out_dtype, ws, need, nullptr, stream);
}

}  // extern "C"

