"""CPU oracle for the weight-only low-bit linear layer  Y = A . D(Wq)^T + b.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The HIP library never calls it,
and the two share no code: no kernels, headers, helpers, tables or constants.

It is written to be read against the pages, not to be fast:

* numbers are IEEE float32 with round-to-nearest-even per operation wherever the
  quantiser or the dequantiser computes, and float64 for the matrix product;
* ties of every rounding to an integer code go to the even neighbour, as the
  offline packer of ``selective_state_update_pairnib.py`` (function
  ``pack_pairnib``) does with ``torch.round``;
* the canonical storage layout is the one the pages describe in words: weights
  [out_features, in_features] row-major (piper-kernels package description,
  section "ConvRot INT8"; OrbitQuant Packed Matmul model card, section "API":
  "row-major codebook indices"), two 4-bit codes per byte with the even element in
  the low nibble (``pack_pairnib``), scales and zero-points one per group along the
  input dimension (AutoRound Kernel package description, section "1. Linear",
  "Example": scale and zp of shape [K/G, N], stored here transposed as [N, K/G]).

Readings where the pages are silent (each also listed in the design notes):

* INT4 symmetric: s = fp16(amax/7), q = clamp(rint(w/s), -8, 7), stored as a
  two's-complement nibble (sign extension as in ``dequant_pairnib``).
* INT4 asymmetric ("asym", "+zp" in the AutoRound Kernel tables): w = s (q - z),
  q, z in [0, 15]; lo = min(min w, 0), hi = max(max w, 0), s = fp16((hi - lo)/15),
  z = clamp(rint(-lo/s), 0, 15), q = clamp(rint(w/s) + z, 0, 15).
* INT8 group 256 with bf16 scales (piper-kernels, "ConvRot INT8": ``group_size=256``,
  ``logical_dtype=torch.bfloat16``): s = bf16(amax/127), q = clamp(rint(w/s), -127, 127)
  (the INT8 convention of ``pack_pairnib``: amax/127 and +-127).
* Every scale is rounded to its storage type first and the codes are computed with
  the stored scale, so weights already on the grid reproduce exactly.
* An all-zero group gets scale 0 and codes 0 (zero-point 0); an all-zero MXFP4 block
  gets scale code 127 (1.0).
* MXFP4: E2M1 elements (sign, two exponent bits with bias 1, one mantissa bit) and one
  E8M0 scale 2^(c-127) per 32 inputs, as in the OCP Microscaling (MX) v1.0
  specification; the pages name the format (Petit package description, "Features";
  AutoRound Kernel "Supported Data Types": FP4 (E2M1), E8M0 scales) but do not
  define it.  Scale exponent e = floor(log2 amax) - 2, read from the float32
  exponent, clamped to [-127, 127]; elements w / 2^e rounded to the nearest E2M1
  value, ties to the even code, saturating at +-6; -0 is stored as +0 (Petit,
  "Known limitations": no negative zeros, positive scales).
* 4-bit codebook (OrbitQuant card, "API"): bf16 row norms, float32 centroids
  [16] of a Lloyd-Max quantiser of N(0,1).  norm_n = bf16(||W_n||_2) (sum of
  squares and square root in float64, one rounding); u = w * fp32(sqrt K) / norm_n;
  idx = nearest centroid, ties to the lower index; decode w = fp32(c[idx]) * s_n
  with s_n = fp32(norm_n) / fp32(sqrt K).
* SwiGLU input [.., 2K] = [up | gate], h = up * silu(gate) (piper-kernels,
  "ConvRot INT8"), evaluated in float64 and rounded once to bf16, i.e. the
  activation is materialised in the activation dtype before the linear.
* Bias is bf16 [N], added before the final rounding; the reference output is the
  exact float64 Y, from which the bf16 output is one rounding away.
* INT8 low-rank merge (piper-kernels, "ConvRot INT8", ``addmm_``): W <- beta W +
  alpha (mat1 @ mat2), then requantised.  mat1 [N, r] and mat2 [r, K] are bf16; the
  product's inner sum runs in index order as float32 fused multiply-adds (each step
  d <- fp32(d + a*b) with the exact product, one rounding), then beta*W and
  alpha*(mat1 @ mat2) are rounded to float32 and summed with one more rounding.  The group scales are
  recomputed by the deterministic RTN rule above; without a seed the codes are RTN, with
  a 64-bit seed each value v = w/s takes floor(v) + 1 with probability v - floor(v)
  (the distance to floor(v)), else floor(v), by comparing that distance with a 24-bit
  uniform drawn from SplitMix64 at counter n*K + k.
* INT8-compute path (AutoRound Kernel, "1. Linear": W4A8 / W8A8 with dynamic activation
  quantisation, QQQ-style): each activation row is quantised symmetrically with its own
  float32 scale s_m = amax_m / 127 and codes clamp(rint(x / s_m), -127, 127); the output
  is the exact product of those dequantised activations with D(Wq).
"""
from __future__ import annotations

import math

import numpy as np
from scipy import special

FORMATS = ("int4", "mxfp4", "int8", "cb4")

# --------------------------------------------------------------------------------------
# Scalar number formats
# --------------------------------------------------------------------------------------


def bf16_round(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); result as float32.

    bf16 keeps the float32 sign and exponent and the top 7 fraction bits, so the
    rounding acts on the low 16 bits of the float32 encoding.  NaN stays NaN."""
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    rest = u & np.uint64(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))
    r = ((keep + up.astype(np.uint64)) << np.uint64(16)).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(a), a, r).astype(np.float32)


def bf16_from_f64(x) -> np.ndarray:
    """Round float64 values directly to bf16 (one rounding, ties to even)."""
    a = np.array(x, dtype=np.float64)
    fin = np.isfinite(a) & (a != 0)
    _, e = np.frexp(a[fin])            # |a| in [2^(e-1), 2^e)
    # bf16 keeps 8 significant bits: spacing 2^(e-8); below the normal range
    # (|a| < 2^-126) the spacing stays 2^-133.
    q = np.maximum(e, -125) - 8
    a[fin] = np.ldexp(np.rint(np.ldexp(a[fin], -q)), q)
    with np.errstate(over="ignore"):
        return a.astype(np.float32)    # exact (<= 8 significant bits) or +-inf


def bf16_bits(x) -> np.ndarray:
    """uint16 encoding of bf16-valued float32 data."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(u) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def fp16_round(x) -> np.ndarray:
    """float32 -> float16, nearest with ties to even (IEEE conversion)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 code (bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa) -> float32.

    Exponent field 0 is subnormal: 0.5 * m.  Otherwise 2^(e-1) * (1 + m/2)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    s = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return (s * mag).astype(np.float32)


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale code c -> 2^(c-127) as float32 (c = 255 is NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    with np.errstate(over="ignore"):
        v = np.ldexp(np.float32(1.0), (c - 127).astype(np.int32)).astype(np.float32)
    return np.where(c == 255, np.float32(np.nan), v).astype(np.float32)


# --------------------------------------------------------------------------------------
# Round-to-nearest quantisers (fp32 arithmetic, RNE), canonical codes out
# --------------------------------------------------------------------------------------


def _groups(w: np.ndarray, group: int) -> np.ndarray:
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    return w.reshape(N, K // group, group)


def quantize_int4_sym(w, group: int):
    """-> (codes int8 [N,K] in [-8,7], scales float16 [N,K/G])."""
    wg = _groups(np.asarray(w, dtype=np.float32), group)
    amax = np.max(np.abs(wg), axis=2)
    s16 = fp16_round(amax / np.float32(7.0))
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(wg / np.where(s > 0, s, np.float32(1))), 0)
    q = np.clip(q, -8, 7).astype(np.int8)
    return q.reshape(w.shape), s16


def quantize_int4_asym(w, group: int):
    """-> (codes uint8 [N,K] in [0,15], scales float16 [N,K/G], zeros uint8 [N,K/G])."""
    wg = _groups(np.asarray(w, dtype=np.float32), group)
    lo = np.minimum(np.min(wg, axis=2), np.float32(0))
    hi = np.maximum(np.max(wg, axis=2), np.float32(0))
    s16 = fp16_round((hi - lo) / np.float32(15.0))
    s = s16.astype(np.float32)
    ok = s > 0
    sd = np.where(ok, s, np.float32(1))
    z = np.where(ok, np.clip(np.rint(-lo / sd), 0, 15), 0).astype(np.float32)
    q = np.where(ok[..., None], np.clip(np.rint(wg / sd[..., None]) + z[..., None], 0, 15), 0)
    return q.astype(np.uint8).reshape(w.shape), s16, z.astype(np.uint8)


def quantize_int8(w, group: int = 256):
    """-> (codes int8 [N,K] in [-127,127], scales: bf16-valued float32 [N,K/G])."""
    wg = _groups(np.asarray(w, dtype=np.float32), group)
    amax = np.max(np.abs(wg), axis=2)
    s = bf16_round(amax / np.float32(127.0))
    ok = s > 0
    sd = np.where(ok, s, np.float32(1))[..., None]
    q = np.where(ok[..., None], np.clip(np.rint(wg / sd), -127, 127), 0)
    return q.astype(np.int8).reshape(w.shape), s


_E2M1_MAG = e2m1_decode(np.arange(8)).astype(np.float64)   # 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_nearest(v) -> np.ndarray:
    """Nearest E2M1 code to each real v (ties to the even code, saturating at +-6,
    -0 stored as +0)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    d = np.abs(a[..., None] - _E2M1_MAG)              # distance to each magnitude
    best = np.argmin(d, axis=-1)                       # first minimum: the lower code
    dmin = np.take_along_axis(d, best[..., None], -1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    dn = np.take_along_axis(d, nxt[..., None], -1)[..., 0]
    tie = (nxt != best) & (dn == dmin) & (best % 2 == 1)
    mag = np.where(tie, nxt, best)
    sign = (v < 0) & (mag != 0)
    return (mag + 8 * sign).astype(np.uint8)


def quantize_mxfp4(w):
    """-> (codes uint8 [N,K] E2M1 in 0..15, scale codes uint8 E8M0 [N,K/32])."""
    wg = _groups(np.asarray(w, dtype=np.float32), 32)
    amax = np.max(np.abs(wg), axis=2)
    _, ex = np.frexp(amax)                      # amax = m 2^ex, m in [0.5, 1)
    e = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)   # floor(log2 amax) - 2
    e = np.where(amax > 0, e, 0)
    v = np.ldexp(wg.astype(np.float64), -e[..., None])    # exact power-of-two scaling
    codes = e2m1_nearest(v)
    return codes.reshape(w.shape), (e + 127).astype(np.uint8)


def lloyd_max_gaussian(levels: int = 16, tol: float = 1e-15, iters: int = 200000):
    """Lloyd-Max quantiser of the standard normal density (OrbitQuant card: "Lloyd-Max
    centroids").  Alternates the two optimality conditions: thresholds at midpoints
    of neighbouring centroids, centroids at the conditional mean of their cell,
    E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    Returns (centroids float64 [levels] ascending, thresholds float64 [levels-1])."""
    half = levels // 2
    c = np.linspace(0.1, 2.5, half)                     # positive half; symmetric
    phi = lambda t: np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)
    for _ in range(iters):
        t = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        lo, hi = t[:-1], t[1:]
        mass = special.ndtr(hi) - special.ndtr(lo)
        new = (phi(lo) - np.where(np.isinf(hi), 0.0, phi(hi))) / mass
        if np.max(np.abs(new - c)) < tol:
            c = new
            break
        c = new
    cent = np.concatenate((-c[::-1], c))
    thr = 0.5 * (cent[:-1] + cent[1:])
    return cent, thr


def _bf16_value(bits: int) -> float:
    """Value of a non-negative bf16 bit pattern; the pattern after the largest finite
    value (the infinity) stands for 2^128, the next power of two, so that the midpoint
    between them is the overflow threshold of round-to-nearest."""
    if bits >= 0x7F80:
        return 2.0 ** 128
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def row_norm_bf16(w) -> np.ndarray:
    """bf16 of the exact Euclidean norm of each row, rounded once (nearest, ties to the
    even bf16 value): the norm that no summation order changes.

    The square of a float32 value is exact in float64, and math.fsum returns the
    correctly rounded float64 s of the exact sum S of the squares.  The bf16 value of
    sqrt(S) is decided by where S lies against the squares of the midpoints m between
    neighbouring bf16 values; a midpoint has 9 significant bits, so m^2 is exact in
    float64.  Rounding is monotonic and m^2 is representable, so s > m^2 implies S > m^2
    and s < m^2 implies S < m^2; only s == m^2 needs S itself, summed in exact rational
    arithmetic.  S == m^2 means sqrt(S) == m: a tie, resolved to the even value."""
    from fractions import Fraction
    w = np.asarray(w, dtype=np.float32)
    out = np.zeros(w.shape[0], dtype=np.float32)
    for n in range(w.shape[0]):
        sq = w[n].astype(np.float64) ** 2
        s = math.fsum(sq)
        if s == 0.0:
            continue
        exact = None

        def cmp(m2: float) -> int:          # sign of S - m2
            nonlocal exact
            if s != m2:
                return 1 if s > m2 else -1
            if exact is None:
                exact = sum((Fraction(float(v)) for v in sq), Fraction(0))
            return (exact > Fraction(m2)) - (exact < Fraction(m2))

        b = int(bf16_bits(bf16_from_f64(np.array([math.sqrt(s)])))[0])   # a neighbour of the answer
        while True:
            hi = 0x7F80 if b >= 0x7F80 else b + 1
            c_hi = -1 if b >= 0x7F80 else cmp(((_bf16_value(b) + _bf16_value(hi)) / 2) ** 2)
            c_lo = 1 if b == 0 else cmp(((_bf16_value(b - 1) + _bf16_value(b)) / 2) ** 2)
            if c_hi > 0 or (c_hi == 0 and b & 1):
                b = hi
            elif c_lo < 0 or (c_lo == 0 and b & 1):
                b = b - 1
            else:
                break
        out[n] = np.inf if b >= 0x7F80 else np.float32(_bf16_value(b))
    return out


def quantize_cb4(w, centroids, norms=None):
    """-> (indices uint8 [N,K] in 0..15, row norms: bf16-valued float32 [N]).

    If ``norms`` is given it is used instead of the computed row norms."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    c32 = np.asarray(centroids, dtype=np.float32)
    if norms is None:
        nrm = row_norm_bf16(w)
    else:
        nrm = np.asarray(norms, dtype=np.float32)
    rk = np.float32(math.sqrt(K))
    ok = nrm > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (w * rk) / np.where(ok, nrm, np.float32(1))[:, None]
    d = np.abs(u.astype(np.float64)[..., None] - c32.astype(np.float64))
    idx = np.argmin(d, axis=-1)                 # first minimum: ties -> lower index
    idx = np.where(ok[:, None], idx, 0)
    return idx.astype(np.uint8), nrm


# --------------------------------------------------------------------------------------
# Canonical packing (two 4-bit codes per byte, even element in the low nibble)
# --------------------------------------------------------------------------------------


def pack_nibbles(codes) -> np.ndarray:
    """codes [N,K] (values taken mod 16, so signed INT4 becomes two's complement)
    -> uint8 [N, K/2] with element 2j in bits 0..3 and element 2j+1 in bits 4..7."""
    c = (np.asarray(codes).astype(np.int64) & 0xF).astype(np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even for 4-bit packing")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    """uint8 [N, K/2] -> uint8 [N, K] nibble values 0..15 (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def sign_extend4(n) -> np.ndarray:
    n = np.asarray(n, dtype=np.int16)
    return (n - 16 * (n > 7)).astype(np.int8)


# --------------------------------------------------------------------------------------
# Dequantisation D(Wq) in float32
# --------------------------------------------------------------------------------------


def _expand(s, group: int) -> np.ndarray:
    return np.repeat(np.asarray(s, dtype=np.float32), group, axis=1)


def dequant_int4(packed, scales16, zeros, group: int) -> np.ndarray:
    """w = s * q (symmetric, q two's complement) or w = s * (q - z) (with zero-point)."""
    n = unpack_nibbles(packed)
    s = _expand(np.asarray(scales16, dtype=np.float16).astype(np.float32), group)
    if zeros is None:
        q = sign_extend4(n).astype(np.float32)
    else:
        q = n.astype(np.float32) - _expand(np.asarray(zeros, dtype=np.float32), group)
    return (q * s).astype(np.float32)


def dequant_int8(codes, scales_bf16, group: int) -> np.ndarray:
    return (np.asarray(codes, dtype=np.int8).astype(np.float32) * _expand(scales_bf16, group)).astype(np.float32)


def dequant_mxfp4(packed, e8m0) -> np.ndarray:
    v = e2m1_decode(unpack_nibbles(packed))
    with np.errstate(over="ignore"):
        return (v * _expand(e8m0_decode(e8m0), 32)).astype(np.float32)


def cb4_row_scale(norms_bf16, K: int) -> np.ndarray:
    """s_n = fp32(norm_n) / fp32(sqrt K) (one float32 division)."""
    return (np.asarray(norms_bf16, dtype=np.float32) / np.float32(math.sqrt(K))).astype(np.float32)


def dequant_cb4(packed, norms_bf16, centroids, K: int) -> np.ndarray:
    idx = unpack_nibbles(packed)
    c = np.asarray(centroids, dtype=np.float32)[idx.astype(np.int64)]
    return (c * cb4_row_scale(norms_bf16, K)[:, None]).astype(np.float32)


# --------------------------------------------------------------------------------------
# Activation stage and the linear
# --------------------------------------------------------------------------------------


def silu64(g) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_bf16(up_gate) -> np.ndarray:
    """Raw input [M, 2K] = [up | gate] -> h = bf16(up * silu(gate)) [M, K]."""
    a = np.asarray(up_gate, dtype=np.float64)
    K = a.shape[-1] // 2
    return bf16_from_f64(a[..., :K] * silu64(a[..., K:]))


def linear_ref(a, dw, bias=None) -> np.ndarray:
    """Y = a . dw^T + b in float64 (a [M,K], dw [N,K], bias [N])."""
    y = np.asarray(a, dtype=np.float64) @ np.asarray(dw, dtype=np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def dequant(fmt: str, canon: dict, K: int) -> np.ndarray:
    """D(Wq) float32 [N, K] from a canonical weight dictionary (see ``quantize``)."""
    if fmt == "int4":
        return dequant_int4(canon["codes"], canon["scales"], canon.get("zeros"), canon["group"])
    if fmt == "mxfp4":
        return dequant_mxfp4(canon["codes"], canon["scales"])
    if fmt == "int8":
        return dequant_int8(canon["codes"], bf16_from_bits(canon["scales"]), canon["group"])
    if fmt == "cb4":
        return dequant_cb4(canon["codes"], bf16_from_bits(canon["scales"]), canon["centroids"], K)
    raise ValueError(fmt)


def quantize(fmt: str, w, group: int = 128, symmetric: bool = True, centroids=None) -> dict:
    """Quantise float32 master weights [N, K] into the canonical layout:

    * int4:  codes uint8 [N,K/2] nibbles, scales float16 [N,K/G], zeros uint8 [N,K/G] | None
    * mxfp4: codes uint8 [N,K/2] nibbles, scales uint8 E8M0 [N,K/32]
    * int8:  codes int8 [N,K],            scales uint16 bf16 bits [N,K/G]
    * cb4:   codes uint8 [N,K/2] nibbles, scales uint16 bf16 norm bits [N], centroids fp32 [16]
    """
    if fmt == "int4":
        if symmetric:
            q, s = quantize_int4_sym(w, group)
            return dict(codes=pack_nibbles(q), scales=s, zeros=None, group=group)
        q, s, z = quantize_int4_asym(w, group)
        return dict(codes=pack_nibbles(q), scales=s, zeros=z, group=group)
    if fmt == "mxfp4":
        q, e = quantize_mxfp4(w)
        return dict(codes=pack_nibbles(q), scales=e, group=32)
    if fmt == "int8":
        q, s = quantize_int8(w, group)
        return dict(codes=q, scales=bf16_bits(s), group=group)
    if fmt == "cb4":
        c = (lloyd_max_gaussian(16)[0] if centroids is None else np.asarray(centroids)).astype(np.float32)
        q, nrm = quantize_cb4(w, c)
        return dict(codes=pack_nibbles(q), scales=bf16_bits(nrm), centroids=c, group=0)
    raise ValueError(fmt)


def forward(fmt: str, x, canon: dict, K: int, bias=None, swiglu: bool = False) -> np.ndarray:
    """Exact reference output Y (float64) for bf16 input x ([M,K], or [M,2K] raw
    SwiGLU input): activation stage, D(Wq), float64 product, bias."""
    a = swiglu_bf16(x) if swiglu else np.asarray(x, dtype=np.float32)
    return linear_ref(a, dequant(fmt, canon, K), bias)


def forward_grouped(fmt: str, x, canons, counts, K: int, N: int, biases=None) -> np.ndarray:
    """Mixture-of-experts linear (AutoRound Kernel package description, "2. MoE
    (Mixture-of-Experts Grouped GEMM)": activations [total_tokens, K], per-expert weights,
    num_tokens_per_expert [E], output [total_tokens, N]).  Tokens are grouped by expert
    in expert order; token t of expert e's slice is multiplied by expert e's D(Wq) and
    bias.  Counts are clipped as the library documents (negative -> 0, nothing past T);
    rows past the sum of the counts are NaN here (the library leaves them untouched)."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    y = np.full((T, N), np.nan, dtype=np.float64)
    run = 0
    for e, c in enumerate(counts):
        c = min(max(int(c), 0), T - run)
        if c:
            b = None if biases is None else biases[e]
            y[run:run + c] = forward(fmt, x[run:run + c], canons[e], K, b)
        run += c
    return y


def output_rows(fmt: str, x, canon: dict, K: int, rows, cols, bias=None, swiglu=False) -> np.ndarray:
    """Y[rows[i], cols[i]] one by one (float64), dequantising only the needed weight
    rows: for sampled checks of large shapes."""
    cols = np.asarray(cols)
    a = swiglu_bf16(np.asarray(x)[np.unique(rows)]) if swiglu else None
    ucols = np.unique(cols)
    sub = {}
    for k, v in canon.items():
        if isinstance(v, np.ndarray) and v.ndim >= 1 and k not in ("centroids",):
            sub[k] = v[ucols]
        else:
            sub[k] = v
    dw = dequant(fmt, sub, K).astype(np.float64)
    pos = {c: i for i, c in enumerate(ucols)}
    rpos = {r: i for i, r in enumerate(np.unique(rows))}
    out = np.empty(len(cols), dtype=np.float64)
    for i, (r, c) in enumerate(zip(rows, cols)):
        arow = a[rpos[r]] if swiglu else np.asarray(x[r], dtype=np.float64)
        out[i] = float(np.dot(arow.astype(np.float64), dw[pos[c]]))
        if bias is not None:
            out[i] += float(bias[c])
    return out


def canonical_bytes(fmt: str, N: int, K: int) -> dict:
    """Storage of the codebook weight path (the accounting of the OrbitQuant card, section
    "Benchmark": packed indices + row norms + centroids)."""
    if fmt != "cb4":
        raise ValueError(fmt)
    return dict(codes=N * K // 2, scales=2 * N, aux=4 * 16)


# --------------------------------------------------------------------------------------
# In-place low-rank update of an INT8 weight with requantisation
# (piper-kernels package description, "ConvRot INT8": ``addmm_`` and ``rounding_seed``)
# --------------------------------------------------------------------------------------

SPLITMIX64_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed, index) -> np.ndarray:
    """Output number ``index`` (0-based) of the SplitMix64 generator seeded with ``seed``.

    SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
    OOPSLA 2014) walks a 64-bit state by the odd constant 0x9E3779B97F4A7C15 (the golden
    ratio times 2^64) and sends each state through a 64-bit finaliser: xor-shift by 30,
    multiply by 0xBF58476D1CE4E5B9, xor-shift by 27, multiply by 0x94D049BB133111EB,
    xor-shift by 31 (Stafford's variant 13 of the MurmurHash3 finaliser).  Output i is
    the finaliser of seed + (i + 1) * gamma, all modulo 2^64, so any output can be had
    directly from its counter."""
    with np.errstate(over="ignore"):
        x = np.asarray(seed, dtype=np.uint64) + (np.asarray(index, dtype=np.uint64) + np.uint64(1)) * \
            np.uint64(SPLITMIX64_GAMMA)
        z = (x ^ (x >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def uniform24(seed, index) -> np.ndarray:
    """The top 24 bits of SplitMix64 output ``index`` as a float32 in [0, 1) (exact)."""
    return (splitmix64(seed, index) >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)


def lowrank_product_f32(mat1, mat2) -> np.ndarray:
    """mat1 @ mat2 (bf16 operands) as a chain of float32 fused multiply-adds in index
    order: d_0 = +0, d_j = fp32(d_{j-1} + mat1[:, j] * mat2[j, :]) with the product exact
    and one rounding per step.

    The product of two bf16 values (8 significant bits each) is exact in float64, and
    so is nothing lost by first rounding d + a*b to float64: rounding a sum of two
    operands of at most 24 significant bits to 53 bits and then to 24 bits gives the
    single rounding to 24 bits (double rounding is innocuous when the first precision
    has at least 2p + 1 bits; S. A. Figueroa, "When is double rounding innocuous?",
    SIGNUM Newsletter 30(3), 1995)."""
    m1 = np.asarray(mat1, dtype=np.float32).astype(np.float64)
    m2 = np.asarray(mat2, dtype=np.float32).astype(np.float64)
    d = np.zeros((m1.shape[0], m2.shape[1]), dtype=np.float32)
    for j in range(m2.shape[0]):
        d = (d.astype(np.float64) + m1[:, j:j + 1] * m2[j:j + 1, :]).astype(np.float32)
    return d


def merge_lowrank_int8(canon: dict, mat1, mat2, alpha=1.0, beta=1.0, seed=None, rows=None) -> dict:
    """INT8 ``addmm_``: W <- beta * D(W) + alpha * (mat1 @ mat2), requantised to INT8 with
    the same group size (piper-kernels, "ConvRot INT8": the update follows the standard
    ``Tensor.addmm_`` contract and requantises; an unsigned 64-bit ``rounding_seed``
    picks one of the two neighbouring INT8 codes at random with probability given by the
    distance, keeps the deterministic scales and draws from no global generator; no seed
    keeps nearest rounding).

    canon: int8 canonical weight (codes int8 [N,K], scales bf16 bits [N,K/G]).
    mat1: bf16-valued [N, r] (the adapter's B); mat2: bf16-valued [r, K] (its A).
    rows: optional row subset (the result then holds only those rows, in that order).
    The random draw for weight (n, k) is ``uniform24(seed, n*K + k)``; the upper code is
    taken when that uniform is below v - floor(v)."""
    G = int(canon["group"])
    codes = np.asarray(canon["codes"], dtype=np.int8)
    N, K = codes.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    w_old = dequant_int8(codes[rows], bf16_from_bits(np.asarray(canon["scales"])[rows]), G)
    d = lowrank_product_f32(np.asarray(mat1, dtype=np.float32)[rows], mat2)
    w = np.float32(beta) * w_old + np.float32(alpha) * d          # float32, three roundings
    if seed is None:
        q, s = quantize_int8(w, G)
        return dict(codes=q, scales=bf16_bits(s), group=G)
    wg = _groups(w, G)
    amax = np.max(np.abs(wg), axis=2)
    s = bf16_round(amax / np.float32(127.0))                       # the deterministic scale
    ok = s > 0
    sd = np.where(ok, s, np.float32(1))[..., None]
    v = wg / sd
    lo = np.floor(v)
    dist = v - lo                                                 # exact in float32
    ctr = rows[:, None].astype(np.uint64) * np.uint64(K) + np.arange(K, dtype=np.uint64)[None, :]
    u = uniform24(seed, ctr).reshape(wg.shape)
    q = lo + (u < dist)
    q = np.where(ok[..., None], np.clip(q, -127, 127), 0)
    return dict(codes=q.astype(np.int8).reshape(w.shape), scales=bf16_bits(s), group=G)


# --------------------------------------------------------------------------------------
# INT8-compute variant: dynamic per-token activation quantisation
# (AutoRound Kernel package description, "1. Linear": "Key Features" W4A8 rescale,
# QQQ-style; "Supported Data Types" note: INT8 compute includes dynamic activation
# quantisation and results are dequantised to floating point)
# --------------------------------------------------------------------------------------


def quantize_activations_int8(x):
    """Per-row symmetric INT8 quantisation of activations [M, K] in float32:
    s_m = fp32(amax_m / 127), q = clamp(rint(x / s_m), -127, 127) (ties to even);
    an all-zero row gets s = 0 and codes 0.  -> (codes int8 [M, K], scales float32 [M])."""
    a = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(a), axis=1) if a.shape[1] else np.zeros(a.shape[0], np.float32)
    s = (amax / np.float32(127.0)).astype(np.float32)
    ok = s > 0
    sd = np.where(ok, s, np.float32(1))[:, None]
    q = np.where(ok[:, None], np.clip(np.rint(a / sd), -127, 127), 0)
    return q.astype(np.int8), s


def forward_a8(fmt: str, x, canon: dict, K: int, bias=None) -> np.ndarray:
    """Exact output (float64) of the INT8-compute linear: the activation rows quantised by
    ``quantize_activations_int8`` and dequantised (codes times row scale), times D(Wq)."""
    q, s = quantize_activations_int8(x)
    a = q.astype(np.float64) * s.astype(np.float64)[:, None]
    return linear_ref(a, dequant(fmt, canon, K), bias)
