/*
 * qlinear.h -- C ABI of the MI355X (gfx950) weight-only low-bit linear layer
 *
 *     Y[M, N] = A[M, K] . D(Wq)[N, K]^T + b[N]
 *
 * A is the bf16 activation X, or h = up * silu(gate) formed from a raw bf16 input
 * [M, 2K] = [up | gate] (piper-kernels 0.2.1 package description, section
 * "ConvRot INT8": convrot_linear(..., input_activation="swiglu") on a [.., 2*in]
 * input).  D(Wq) is the weight decoded from one of four packed formats; it is decoded
 * in registers inside the kernels and never written out as a dense matrix (OrbitQuant
 * Packed Matmul model card, "API": no dequantized weight cache; AutoRound Kernel
 * package description, "1. Linear": woqgemm on a packed blob).
 *
 * Formats (canonical, i.e. checkpoint, layouts; N = out_features, K = in_features):
 *
 *   QL_INT4   codes  uint8 [N, K/2]  two 4-bit codes per byte, even k in the low nibble
 *                                    (selective_state_update_pairnib.py, pack_pairnib);
 *                                    two's complement q in [-8, 7] when symmetric,
 *                                    unsigned q in [0, 15] with a zero-point
 *             scales fp16  [N, K/G]  G in {32, 64, 128, 256}
 *             zeros  uint8 [N, K/G]  0..15, or NULL for symmetric.   w = s*q  or  s*(q - z)
 *             (AutoRound Kernel, "1. Linear", "Example": qweight, scale and zp per group;
 *              "Supported Data Types": sym / asym)
 *   QL_MXFP4  codes  uint8 [N, K/2]  E2M1 codes (sign, 2 exponent bits bias 1, 1 mantissa)
 *             scales uint8 [N, K/32] E8M0 codes c -> 2^(c-127), code 255 = NaN (its
 *                                    block decodes to NaN); G must be 32
 *             (Petit package description, "Features": MXFP4 weights)
 *   QL_INT8   codes  int8  [N, K]    q in [-128, 127]
 *             scales bf16  [N, K/G]  G in {32, 64, 128, 256}; 256 is ConvRot's group
 *             (piper-kernels, "ConvRot INT8": group_size=256, logical_dtype=bfloat16)
 *   QL_CB4    codes  uint8 [N, K/2]  4-bit indices into a 16-entry codebook
 *             scales bf16  [N]       row norms;  w = c[idx] * norm_n / sqrt(K)
 *             aux    fp32  [16]      centroids, symmetric: c[15-j] == -c[j]
 *             (OrbitQuant card, "API": packed indices, row norms, Lloyd-Max centroids)
 *
 * qlinear_pack() shuffles a canonical weight once, offline, into the device layout
 * that the kernels stream with coalesced 16-byte loads (Petit package description,
 * "Techniques and performance": weights shuffled offline so that on-GPU
 * dequantisation is cheap).  qlinear_unpack() inverts it bit-exactly.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless an argument says "host".  The caller
 *     allocates and owns every buffer; the library allocates no device memory and
 *     keeps no device state.  Sizes come from qlinear_packed_bytes() and
 *     qlinear_workspace_bytes().
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is queued
 *     on it asynchronously; no entry point synchronises or copies device memory to
 *     the host.
 *   - Every argument is validated before anything is queued: an error return leaves
 *     all outputs untouched.  QL_E_HIP reports a failed launch.
 *   - Entry points are reentrant; concurrent calls on different streams are safe
 *     when their output buffers do not overlap.
 *   - Device pointers must be 16-byte aligned (x, packed buffers, workspace) or
 *     aligned to their element size (bias, out, canonical arrays).
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QL_OK = 0,
    QL_E_ARG = 1,          /* NULL where a buffer is required, unknown enum value    */
    QL_E_SHAPE = 2,        /* negative size, K not a multiple of 32 or of the group,
                              unsupported group size for the format                  */
    QL_E_ALIGN = 3,        /* a pointer is not aligned as required                    */
    QL_E_UNSUPPORTED = 4,  /* a combination the kernels do not implement (e.g. an
                              asymmetric codebook); never a silent fallback          */
    QL_E_WORKSPACE = 5,    /* workspace smaller than qlinear_workspace_bytes()        */
    QL_E_HIP = 6           /* a HIP launch failed                                     */
} ql_status;

typedef enum { QL_INT4 = 0, QL_MXFP4 = 1, QL_INT8 = 2, QL_CB4 = 3 } ql_format;
typedef enum { QL_ACT_NONE = 0, QL_ACT_SWIGLU = 1 } ql_act;
typedef enum { QL_BF16 = 0, QL_F32 = 1 } ql_dtype;

/* Library version, e.g. 0x000100 for 0.1.0. */
int qlinear_version(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char *qlinear_error_string(ql_status s);

/*
 * Bytes of the three device-layout buffers of a packed weight.
 *   f, N, K, group  as above (group is ignored for QL_CB4 and must be 32 for QL_MXFP4)
 *   has_zeros       1 for INT4 with a zero-point, else 0
 *   w_bytes         packed codes
 *   s_bytes         packed scales (CB4: float32 row scales and bf16 norms)
 *   aux_bytes       packed zero-points (INT4 with zeros), codebook record (CB4, 128 B),
 *                   else 0
 * All three are multiples of 256.  Host-only: touches no device.
 */
ql_status qlinear_packed_bytes(ql_format f, int64_t N, int64_t K, int group, int has_zeros,
                               size_t *w_bytes, size_t *s_bytes, size_t *aux_bytes);

/*
 * Offline pack: canonical arrays -> device layout (one kernel launch per buffer).
 *   codes   canonical codes (see the format table)
 *   scales  canonical scales (CB4: bf16 row norms [N])
 *   aux_in  INT4: zeros uint8 [N, K/G] or NULL (symmetric); CB4: HOST pointer to the 16
 *           float32 centroids, read during the call; otherwise must be NULL
 *   packed_w, packed_s, packed_aux   outputs sized by qlinear_packed_bytes()
 *           (packed_aux may be NULL when aux_bytes is 0)
 * CB4 also chooses a per-codebook multiplier alpha in [1, 2) that minimises the bf16
 * rounding error of alpha * c[j] and records it in packed_aux, together with the
 * matrix-core operand the kernels will use: one bf16 term per level (about 1e-3 relative
 * error, one MFMA per fragment), or two terms hi + lo (about 16 bits, two MFMAs) when the
 * largest row norm exceeds 3 x their rms -- the single term's error is relative to each
 * row's own output, so a dominant row would carry it into the outputs that set the
 * output's rms.  The choice is taken on the device from the norms, once, here.
 * Errors: QL_E_UNSUPPORTED for a codebook that is not symmetric or not finite.
 */
ql_status qlinear_pack(ql_format f, int64_t N, int64_t K, int group,
                       const void *codes, const void *scales, const void *aux_in,
                       void *packed_w, void *packed_s, void *packed_aux, void *stream);

/*
 * On-device round-to-nearest quantiser: dense weights -> the canonical arrays that
 * qlinear_pack() takes (the step before the offline pack: quantising a dense
 * high-precision weight, piper-kernels package description, "ConvRot INT8", from_hp;
 * per-group amax, scale and rint to the grid as the offline packer pack_pairnib of
 * selective_state_update_pairnib.py does).  Every operation is IEEE float32 with
 * round-to-nearest-even, in this order:
 *   INT4 symmetric   s = fp16(amax/7),  q = clamp(rint(w/s), -8, 7)
 *   INT4 asymmetric  lo = min(min w, 0), hi = max(max w, 0), s = fp16((hi-lo)/15),
 *                    z = clamp(rint(-lo/s), 0, 15), q = clamp(rint(w/s) + z, 0, 15)
 *   INT8             s = bf16(amax/127), q = clamp(rint(w/s), -127, 127)
 *   MXFP4            e = floor(log2 amax) - 2 in [-127, 127] (0 for a zero block);
 *                    element = nearest E2M1 value of w * 2^-e (ties to the even code,
 *                    saturating at 6, no negative zero); scale code e + 127
 *   CB4              norm = bf16 of the float64 row norm (one rounding);
 *                    u = (w * fp32(sqrt K)) / norm; index of the nearest level (float64
 *                    distances, ties to the lower index)
 * A scale that rounds to zero gives codes 0 (and zero-point 0).
 *   w          float32 [N, K] row-major (device), finite
 *   group      as for qlinear_pack (CB4: 0)
 *   levels     CB4: HOST pointer to the 16 float32 levels, read during the call; else NULL
 *   codes      out: canonical codes (uint8 [N, K/2] nibbles, even k low; INT8 int8 [N, K])
 *   scales     out: fp16 [N, K/G] (INT4), uint8 E8M0 [N, K/32] (MXFP4),
 *              bf16 [N, K/G] (INT8), bf16 row norms [N] (CB4)
 *   zeros      out: INT4 asymmetric uint8 [N, K/G] (0..15); NULL = symmetric INT4;
 *              must be NULL for the other formats
 * Alignment: w 8 bytes, codes 2 bytes, scales and zeros their element size.
 * Errors: QL_E_SHAPE / QL_E_ARG as for qlinear_pack; QL_E_UNSUPPORTED for
 * non-finite levels.
 */
ql_status qlinear_quantize(ql_format f, int64_t N, int64_t K, int group, const float *w,
                           const float *levels, void *codes, void *scales, void *zeros, void *stream);

/*
 * In-place low-rank update of a packed INT8 weight, requantised into the same buffers
 * (piper-kernels package description, "ConvRot INT8": addmm_ computes
 * weight = beta * weight + alpha * (mat1 @ mat2) with the Tensor.addmm_ contract,
 * requantises and keeps the quantised storage; an unsigned 64-bit rounding seed picks
 * one of the two neighbouring INT8 codes at random with probability set by the distance,
 * without changing the deterministic scales; without a seed, nearest rounding).
 * Every operation is IEEE float32 with one rounding:
 *   w_old = q * s;  d_0 = +0,  d_j = fma(mat1[n, j], mat2[j, k], d_{j-1}) in index order
 *   w = beta * w_old + alpha * d       (the two products rounded, then their sum)
 *   s' = bf16(amax |w| / 127) per group   (the quantiser's INT8 rule, both modes)
 *   v = w / s';  stochastic = 0: code = clamp(rint(v), -127, 127)
 *                stochastic = 1: code = clamp(floor(v) + [u < v - floor(v)], -127, 127),
 *                u = (SplitMix64 output n*K + k of `seed`) >> 40, times 2^-24
 *   (SplitMix64, Steele, Lea and Flood 2014: output i = the 64-bit finaliser of
 *   seed + (i + 1) * 0x9E3779B97F4A7C15).  A scale that rounds to zero gives codes 0.
 *   N, K, group        as packed by qlinear_pack() (INT8)
 *   packed_w, packed_s the weight's device buffers, read and rewritten in place (16-byte
 *                      aligned); padding bytes keep their packed values
 *   mat1               bf16 [N, rank] row-major (device): the adapter's B
 *   mat2               bf16 [rank, K] row-major (device): the adapter's A
 *   rank               0 .. 256 (0: mat1 and mat2 may be NULL; the update is then
 *                      beta * W, requantised)
 *   alpha, beta        finite
 * Repeated updates are lossy, as the page warns: each one requantises.  Two updates of
 * one weight must be ordered (one stream); the merged values must stay finite.
 * Errors: QL_E_SHAPE as for qlinear_pack; QL_E_ARG for null buffers, a rank outside
 * 0 .. 256, stochastic not 0 or 1, or non-finite alpha or beta; QL_E_ALIGN.
 */
ql_status qlinear_int8_addmm(int64_t N, int64_t K, int group, void *packed_w, void *packed_s,
                             const void *mat1, const void *mat2, int64_t rank, float alpha, float beta,
                             int stochastic, uint64_t seed, void *stream);

/*
 * Inverse of qlinear_pack(): device layout -> canonical arrays, bit-exact (AutoRound
 * Kernel package description, "1. Linear": unpack_weight recovers the weight from the
 * packed blob, for verification).
 *   codes, scales   canonical outputs
 *   aux_out         INT4 with zeros: zeros [N, K/G]; CB4: float32 centroids [16]
 *                   (device); otherwise NULL
 *   has_zeros       INT4 only: 1 if packed_aux holds zero-points
 */
ql_status qlinear_unpack(ql_format f, int64_t N, int64_t K, int group, int has_zeros,
                         const void *packed_w, const void *packed_s, const void *packed_aux,
                         void *codes, void *scales, void *aux_out, void *stream);

/*
 * Debug dump of a dequantised weight tile, decoded by the same register-level code
 * the GEMM kernels use (AutoRound Kernel package description, "1. Linear":
 * unpack_weight dequantises the packed blob to a dense weight, for verification; here
 * a tile of it at a time).
 *   n0, k0, tn, tk  tile origin and extent (0 <= n0, n0+tn <= N, same for k)
 *   mode 0          out = D(Wq)[n0.., k0..] in float32, exactly as the format defines it
 *   mode 1          out = the bf16 operand the matrix cores receive, widened to float32
 *                   (before group, zero-point and codebook row scaling; a two-term
 *                   codebook operand as the float32 sum hi + lo, which is exact)
 *   out             float32 [tn, tk] row-major
 */
ql_status qlinear_dequant_tile(ql_format f, int64_t N, int64_t K, int group, int has_zeros,
                               const void *packed_w, const void *packed_s, const void *packed_aux,
                               int64_t n0, int64_t k0, int64_t tn, int64_t tk, int mode,
                               float *out, void *stream);

/*
 * Workspace that qlinear_forward() needs for this shape; 0 when no split of the input
 * dimension over workgroups is scheduled.  Host-only (the schedule is a pure function
 * of the shape, fixed for the 256 compute units of gfx950).
 *
 * The workspace holds float32 split-K partial sums (tile schedules) and the bf16 SwiGLU
 * input h when a prologue materialises it (act = SWIGLU, except decode schedules with
 * M <= 2, whose kernel forms h itself).  Its contents on entry do not matter and are
 * overwritten; calls that run at the same time must not share one.
 */
ql_status qlinear_workspace_bytes(ql_format f, int64_t M, int64_t N, int64_t K, int group,
                                  ql_act act, size_t *bytes);

/*
 * The linear layer.
 *   x          bf16 [M, K] (act = NONE) or [M, 2K] = [up | gate] (act = SWIGLU), row-major,
 *              16-byte aligned
 *   M          rows (0 is a no-op); N, K, group, has_zeros as packed
 *   packed_w, packed_s, packed_aux   from qlinear_pack() (packed_aux may be NULL for INT4
 *              without zero-points, INT8 and MXFP4)
 *   bias       bf16 [N] or NULL
 *   out        [M, N] row-major, bf16 (round to nearest even of the float32 result) or
 *              float32 (the same float32 result)
 *   workspace  at least qlinear_workspace_bytes() bytes, 256-byte aligned (NULL if 0)
 * Schedules: for M <= 16 one workgroup per block of output columns streams the whole
 * input dimension, split over its wavefronts and reduced in LDS; larger M uses tiles of
 * 32 to 128 rows with activations and packed weights staged through LDS, split over
 * workgroups when the column blocks alone do not fill the device.  Every schedule
 * accumulates in float32 and adds partial sums in a fixed order, so repeated calls give
 * bit-identical results.  The SwiGLU input is formed by a one-pass prologue, or inside
 * the decode kernel for M <= 2; both give the same h, so the fused and the materialised
 * paths give the same linear (piper-kernels, "ConvRot INT8").
 */
ql_status qlinear_forward(const void *x, int64_t M, int64_t N, int64_t K,
                          const void *packed_w, const void *packed_s, const void *packed_aux,
                          ql_format f, int group, int has_zeros,
                          const void *bias, ql_act act, void *out, ql_dtype out_dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * qlinear_forward() without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments, validation, kernels and results are those of
 * qlinear_forward(), bit for bit; the workspace is a device array of the library,
 * qlinear_noalloc_scratch_bytes() bytes (64 MiB), one copy per GPU, held from the
 * library's load until the process ends.  The call allocates nothing.
 *   - Shapes whose workspace (qlinear_workspace_bytes()) exceeds the scratch are refused
 *     with QL_E_WORKSPACE before any launch.
 *   - The stream must belong to the current device (QL_E_HIP otherwise); the scratch's
 *     device address is looked up on the first call on each device.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last call's
 *     contents (no call depends on them): calls that may overlap on one GPU (two
 *     streams, two threads) race on it and must be ordered by the caller.
 */
size_t qlinear_noalloc_scratch_bytes(void);
ql_status qlinear_forward_noalloc(const void *x, int64_t M, int64_t N, int64_t K,
                                  const void *packed_w, const void *packed_s, const void *packed_aux,
                                  ql_format f, int group, int has_zeros,
                                  const void *bias, ql_act act, void *out, ql_dtype out_dtype,
                                  void *stream);

/*
 * Explicit schedules, for tuning.  CDNA kernels are sensitive to tile shapes (Petit
 * package description, "Known limitations"), so the schedule that qlinear_forward()
 * picks can be inspected and overridden.
 *   tile    index of a compiled tile shape, 0 .. qlinear_num_tiles()-1, or -1 = automatic
 *   splits  tile schedules: number of workgroups along the input dimension, or 0 =
 *           automatic (rounded so that every split holds whole groups).  Decode
 *           schedules split the input dimension over the wavefronts of one workgroup
 *           and take splits 0 or 1; they serve M <= 16 only (QL_E_UNSUPPORTED
 *           otherwise)
 * A schedule whose launch grid exceeds the device's limits (more than 65535 splits) is
 * refused with QL_E_UNSUPPORTED before any launch.
 */
typedef struct ql_schedule {
    int32_t tile;
    int32_t splits;
} ql_schedule;

/* Number of compiled schedules, and for each the rows x columns of output of one
 * workgroup and the inputs it stages per barrier (0 for decode schedules, whose
 * wavefronts stream their own chunks without a workgroup barrier). */
int qlinear_num_tiles(void);
ql_status qlinear_tile_shape(int tile, int *rows, int *cols, int *kblock);

/* The schedule qlinear_forward() uses for a shape (host-only). */
ql_status qlinear_default_schedule(ql_format f, int64_t M, int64_t N, int64_t K, int group,
                                   ql_act act, ql_schedule *out);

/* Workspace bytes for an explicit schedule (NULL = automatic). */
ql_status qlinear_workspace_bytes_ex(ql_format f, int64_t M, int64_t N, int64_t K, int group,
                                     ql_act act, const ql_schedule *sched, size_t *bytes);

/* qlinear_forward() with an explicit schedule (NULL = automatic). */
ql_status qlinear_forward_ex(const void *x, int64_t M, int64_t N, int64_t K,
                             const void *packed_w, const void *packed_s, const void *packed_aux,
                             ql_format f, int group, int has_zeros,
                             const void *bias, ql_act act, void *out, ql_dtype out_dtype,
                             void *workspace, size_t workspace_bytes, const ql_schedule *sched,
                             void *stream);

/*
 * INT8-compute variant (W4A8 / W8A8; AutoRound Kernel package description, "1. Linear":
 * "Key Features", W4A8 / W2A8 rescale in the style of QQQ, low-bit weights re-scaled to
 * INT8 and computed by an INT8 GEMM; "Supported Data Types": INT8 compute includes dynamic
 * activation quantisation, results dequantised to floating point).
 *
 * qlinear_quantize_activations: per-row symmetric INT8 quantisation of bf16 activations,
 * IEEE float32 with round-to-nearest-even: s_m = amax_m / 127,
 * q = clamp(rint(x / s_m), -127, 127); an all-zero row gets s = 0 and codes 0.
 *   x       bf16 [M, K] (device, 16-byte aligned), K a multiple of 32
 *   codes   out: int8 [M, K] (8-byte aligned)      scales  out: float32 [M]
 *
 * qlinear_forward_a8: Y = (q * s) . D(Wq)^T + bias, with q and s as above, computed on
 * the INT8 matrix cores: exact int32 sums per weight group, group scale and row scale
 * in float32, then bias and the output rounding.  Weights: symmetric INT4 (no
 * zero-points) or INT8, packed by qlinear_pack(), group 64, 128 or 256.
 *   workspace   qlinear_a8_workspace_bytes() bytes, 256-byte aligned: the quantised
 *               rows (in the kernel's input order) and their scales are written there
 *   tile        -1: automatic; else 0 .. qlinear_a8_num_tiles() - 1
 * Errors: QL_E_UNSUPPORTED for other formats, zero-points or group 32; otherwise as for
 * qlinear_forward().  M = 0 is a no-op.
 */
ql_status qlinear_quantize_activations(const void *x, int64_t M, int64_t K, void *codes, float *scales,
                                        void *stream);
ql_status qlinear_a8_workspace_bytes(ql_format f, int64_t M, int64_t N, int64_t K, int group, size_t *bytes);
int qlinear_a8_num_tiles(void);
ql_status qlinear_a8_tile_shape(int tile, int *rows, int *cols);
ql_status qlinear_forward_a8(const void *x, int64_t M, int64_t N, int64_t K, const void *packed_w,
                             const void *packed_s, ql_format f, int group, const void *bias, void *out,
                             ql_dtype out_dtype, void *workspace, size_t workspace_bytes, int tile,
                             void *stream);

/*
 * Grouped (mixture-of-experts) linear: every token is multiplied by its own expert's
 * packed weight (AutoRound Kernel package description, "2. MoE (Mixture-of-Experts Grouped
 * GEMM)": activations [total_tokens, K], per-expert weights, num_tokens_per_expert [E]
 * int32, output [total_tokens, N]; Petit package description, "Features": fused MoE
 * kernels for MXFP4 weights).  Tokens are grouped by expert in expert order: expert e
 * owns rows offsets[e] .. offsets[e+1]-1 of x and out, offsets being the running sum of
 * tokens_per_expert.
 *   x                  bf16 [T, K] (device, 16-byte aligned)
 *   tokens_per_expert  int32 [E] (device); read by the device, so it may be computed on
 *                      the device in the same stream.  A negative count counts as 0 and
 *                      counts past T are clipped, so no row beyond T is read or written;
 *                      rows past the sum of the counts are left untouched.
 *   packed_w/s/aux     E experts' packed buffers back to back: expert e's buffers start
 *                      e * w_bytes (s_bytes, aux_bytes) in, with the sizes that
 *                      qlinear_packed_bytes() gives for one expert [N, K]
 *   bias               NULL or bf16 [E, N] (one row per expert)
 *   out                [T, N] bf16 or float32
 *   workspace          qlinear_grouped_workspace_bytes() bytes, 256-byte aligned (the
 *                      expert offsets and the tile map are written there)
 * The kernels are those of qlinear_forward(): the decode kernel in slots of 16 rows when
 * the experts average at most 16 tokens (and ceil(T / 16) + E <= 65535, the grid
 * dimension that holds the slots), else the LDS-ring tiles; each workgroup takes one
 * row block of one expert.  T = 0 or E = 0 is a no-op.  Shapes whose grid would exceed
 * 2^31 - 1 workgroups are refused with QL_E_SHAPE by both functions.
 */
ql_status qlinear_grouped_workspace_bytes(ql_format f, int64_t T, int64_t E, int64_t N, int64_t K,
                                          int group, size_t *bytes);
ql_status qlinear_grouped_forward(const void *x, int64_t T, const int32_t *tokens_per_expert,
                                  int64_t E, int64_t N, int64_t K,
                                  const void *packed_w, const void *packed_s, const void *packed_aux,
                                  ql_format f, int group, int has_zeros, const void *bias,
                                  void *out, ql_dtype out_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
