"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a printed or
textbook value, a closed form, an exhaustive enumeration, an exact rational
computation, an independent library routine, or an invariant that a dropped term,
a wrong sign, a wrong index or a transposed operand would break."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synthetic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------- formats

def test_e2m1_table_exhaustive():
    table = {int(c): float(v) for c, v in _golden("e2m1_values.txt")}
    got = O.e2m1_decode(np.arange(16))
    for c in range(16):
        assert got[c] == table[c]
        assert math.copysign(1.0, got[c]) == math.copysign(1.0, table[c]) or table[c] == 0.0
    # the value set of the format
    assert sorted(set(np.abs(got).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e8m0_all_codes_closed_form():
    got = O.e8m0_decode(np.arange(256))
    for c in range(255):
        assert Fraction(float(got[c])) == Fraction(2) ** (c - 127)
    assert np.isnan(got[255])


def test_bf16_round_matches_torch_and_ties_to_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3.39e38, 0.0, -0.0], dtype=np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.bf16_round(x).view(np.uint32), ref.view(np.uint32))
    # hand ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1); 1 + 3*2^-8 -> 1 + 2^-6
    assert O.bf16_round(np.float32(1 + 2 ** -8)) == 1.0
    assert O.bf16_round(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)


def test_bf16_from_f64_single_rounding():
    # A float64 just above a bf16 midpoint must round up; rounding through float32 first
    # would land on the midpoint and round to even (down).
    x = 1 + 2 ** -8 + 2 ** -40
    assert O.bf16_from_f64(np.array([x]))[0] == np.float32(1 + 2 ** -7)
    assert O.bf16_from_f64(np.array([1 + 2 ** -8]))[0] == 1.0
    assert O.bf16_from_f64(np.array([-1.4621171572600098]))[0] == np.float32(-1.4609375)
    assert O.bf16_from_f64(np.array([2.0 ** -133]))[0] == np.float32(2.0 ** -133)
    assert np.isinf(O.bf16_from_f64(np.array([3.5e38]))[0])
    rng = np.random.default_rng(1)
    v = rng.standard_normal(5000) * 3
    # float64 -> bf16 equals float64 -> exact rational rounding by brute force
    for t in v[:300]:
        r = float(O.bf16_from_f64(np.array([t]))[0])
        m, e = math.frexp(t)
        lo = math.ldexp(math.floor(math.ldexp(t, 8 - e)), e - 8)
        hi = lo + math.ldexp(1.0, e - 8)
        assert r in (lo, hi)
        d_lo, d_hi = abs(Fraction(t) - Fraction(lo)), abs(Fraction(hi) - Fraction(t))
        assert (r == lo and d_lo <= d_hi) or (r == hi and d_hi <= d_lo)


# ----------------------------------------------------------------------------- packing

def test_nibble_order_from_pairnib_packer():
    # selective_state_update_pairnib.py, pack_pairnib: byte = even | (odd << 4)
    assert O.pack_nibbles(np.array([[1, 2, 15, 0]])).tolist() == [[0x21, 0x0F]]
    assert O.pack_nibbles(np.array([[-1, -8, 7, -2]])).tolist() == [[0x8F, 0xE7]]


def test_nibble_roundtrip_exhaustive():
    allbytes = np.arange(256, dtype=np.uint8).reshape(4, 64)
    assert np.array_equal(O.pack_nibbles(O.unpack_nibbles(allbytes)), allbytes)
    rng = np.random.default_rng(2)
    c = rng.integers(0, 16, size=(37, 512))
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(c)), c)
    s = rng.integers(-8, 8, size=(5, 64))
    assert np.array_equal(O.sign_extend4(O.unpack_nibbles(O.pack_nibbles(s))), s)


# ----------------------------------------------------------------------------- INT4

def test_int4_sym_worked_example():
    g = np.zeros(128, dtype=np.float32)
    g[:3] = [0.7, -0.35, 0.1]
    q, s = O.quantize_int4_sym(g[None, :], 128)
    s32 = np.float32(np.float16(np.float32(0.7) / np.float32(7)))
    assert s[0, 0] == np.float16(s32)
    assert q[0, 0] == 7 and q[0, 1] == round(-0.35 / float(s32)) and q[0, 2] == 1
    # exact ties of w/s round to the even integer
    w = np.zeros((1, 128), dtype=np.float32)
    s0 = np.float32(0.125)
    w[0, :5] = np.array([7, 2.5, 3.5, -2.5, 0.5], dtype=np.float32) * s0
    q, s = O.quantize_int4_sym(w, 128)
    assert s[0, 0] == np.float16(0.125)
    assert q[0, :5].tolist() == [7, 2, 4, -2, 0]


def test_int4_sym_on_grid_exact():
    rng = np.random.default_rng(3)
    N, K, G = 16, 512, 128
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    q[:, ::G] = rng.choice([-7, 7], size=(N, K // G))        # every group reaches |q| = 7
    s = (rng.uniform(1e-3, 1e-1, (N, K // G))).astype(np.float16)
    w = O.dequant_int4(O.pack_nibbles(q), s, None, G)
    q2, s2 = O.quantize_int4_sym(w, G)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_int4_asym_on_grid_exact_and_formula():
    rng = np.random.default_rng(4)
    N, K, G = 16, 512, 128
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    q[:, 0::G] = 0
    q[:, 1::G] = 15                                   # each group spans the full code range
    z = rng.integers(0, 16, size=(N, K // G)).astype(np.uint8)
    s = (rng.uniform(1e-3, 1e-1, (N, K // G))).astype(np.float16)
    w = O.dequant_int4(O.pack_nibbles(q), s, z, G)
    # w = s (q - z), checked element by element with exact rationals
    for (n, k) in [(0, 0), (3, 129), (15, 511), (7, 200)]:
        assert Fraction(float(w[n, k])) == Fraction(float(s[n, k // G])) * (int(q[n, k]) - int(z[n, k // G]))
    q2, s2, z2 = O.quantize_int4_asym(w, G)
    assert np.array_equal(q2, q) and np.array_equal(s2, s) and np.array_equal(z2, z)


def test_int4_rtn_error_bound_and_zero_group():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((8, 1024)).astype(np.float32) * np.float32(0.02)
    w[3, 128:256] = 0.0
    q, s = O.quantize_int4_sym(w, 128)
    d = O.dequant_int4(O.pack_nibbles(q), s, None, 128)
    step = np.repeat(s.astype(np.float32), 128, axis=1)
    assert np.all(np.abs(d - w) <= step / 2 * (1 + 1e-6) + 1e-12)
    assert s[3, 1] == 0 and np.all(q[3, 128:256] == 0)
    assert q.min() >= -8 and q.max() <= 7
    qa, sa, za = O.quantize_int4_asym(w, 128)
    da = O.dequant_int4(O.pack_nibbles(qa), sa, za, 128)
    step = np.repeat(sa.astype(np.float32), 128, axis=1)
    assert np.all(np.abs(da - w) <= step / 2 * (1 + 1e-3) + 1e-12)
    assert sa[3, 1] == 0 and za[3, 1] == 0 and np.all(qa[3, 128:256] == 0)


# ----------------------------------------------------------------------------- INT8

def test_int8_on_grid_exact_and_bound():
    rng = np.random.default_rng(6)
    N, K, G = 8, 1024, 256
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    q[:, ::G] = rng.choice([-127, 127], size=(N, K // G))
    s = O.bf16_round(rng.uniform(1e-4, 1e-2, (N, K // G)).astype(np.float32))
    w = O.dequant_int8(q, s, G)
    q2, s2 = O.quantize_int8(w, G)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    w = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.015)
    q, s = O.quantize_int8(w, G)
    d = O.dequant_int8(q, s, G)
    assert np.all(np.abs(d - w) <= np.repeat(s, G, axis=1) * 0.5000001 + 1e-12)
    assert q.min() >= -127


# ----------------------------------------------------------------------------- MXFP4

def test_mxfp4_element_rounding_ties_and_saturation():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.1, -0.25, -0.3, 5.01, 0.2499])
    codes = O.e2m1_nearest(v)
    assert O.e2m1_decode(codes).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 0.0, 0.0, -0.5, 6.0, 0.0]
    assert codes[9] == 0 and codes[10] == 0         # no negative zero


def test_mxfp4_scale_rule_closed_form():
    for amax, e in [(1.0, -2), (0.02, -8), (6.0, 0), (7.99, 0), (8.0, 1), (2.0 ** -130, -127)]:
        w = np.zeros((1, 32), dtype=np.float32)
        w[0, 5] = amax
        _, sc = O.quantize_mxfp4(w)
        assert int(sc[0, 0]) - 127 == e, (amax, sc)
    _, sc = O.quantize_mxfp4(np.zeros((1, 32), dtype=np.float32))
    assert sc[0, 0] == 127


def test_mxfp4_on_grid_exact():
    rng = np.random.default_rng(7)
    N, K = 8, 256
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    q[q == 8] = 0                                       # no negative zero
    q[:, ::32] = rng.choice([6, 7, 14, 15], size=(N, K // 32))  # each block reaches |4| or |6|
    e = rng.integers(100, 140, size=(N, K // 32)).astype(np.uint8)
    w = O.dequant_mxfp4(O.pack_nibbles(q), e)
    q2, e2 = O.quantize_mxfp4(w)
    assert np.array_equal(q2, q) and np.array_equal(e2, e)


def test_mxfp4_nearest_is_brute_force_nearest():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    q, e = O.quantize_mxfp4(w)
    d = O.dequant_mxfp4(O.pack_nibbles(q), e).astype(np.float64)
    sc = np.repeat(O.e8m0_decode(e).astype(np.float64), 32, axis=1)
    grid = np.array(sorted(set(O.e2m1_decode(np.arange(16)).tolist())))
    for n, k in zip(rng.integers(0, 16, 400), rng.integers(0, 256, 400)):
        cand = grid * sc[n, k]
        best = np.min(np.abs(cand - w[n, k]))
        assert abs(d[n, k] - w[n, k]) == best


# ----------------------------------------------------------------------------- codebook

def test_lloyd_max_matches_max_1960_table():
    c, t = O.lloyd_max_gaussian(16)
    gold = _golden("lloyd_max_gaussian_16.txt")
    # one unit in the last printed digit of the table
    ulp = lambda v: 10.0 ** -len(v.split(".")[1])
    lv = [(float(v), ulp(v)) for k, _, v in gold if k == "level"]
    th = [(float(v), ulp(v)) for k, _, v in gold if k == "threshold"]
    mse_tab = [float(v) for k, _, v in gold if k == "mse"][0]
    assert all(abs(a - v) <= u for a, (v, u) in zip(c[8:], lv))
    assert all(abs(a - v) <= u for a, (v, u) in zip(t[7:], th))
    assert np.array_equal(c[:8], -c[8:][::-1])                   # symmetric
    from scipy import integrate, stats
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    mse = 0.0
    for i in range(16):
        a, b = edges[i], edges[i + 1]
        mass = stats.norm.cdf(b) - stats.norm.cdf(a)
        mean = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b)[0] / mass
        assert abs(mean - c[i]) < 1e-9                              # centroid condition
        mse += integrate.quad(lambda x: (x - c[i]) ** 2 * stats.norm.pdf(x), a, b)[0]
    assert abs(mse - mse_tab) < 1e-5


def test_cb4_requantise_with_norms_and_ties():
    c = O.lloyd_max_gaussian(16)[0].astype(np.float32)
    rng = np.random.default_rng(9)
    N, K = 12, 256
    idx = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    nrm = O.bf16_round(rng.uniform(0.1, 2.0, N).astype(np.float32))
    w = O.dequant_cb4(O.pack_nibbles(idx), nrm, c, K)
    i2, n2 = O.quantize_cb4(w, c, norms=nrm)
    assert np.array_equal(i2, idx) and np.array_equal(n2, nrm)
    # decode formula w = c[idx] * norm / sqrt(K) with float32 steps
    s = np.float32(nrm[3]) / np.float32(math.sqrt(K))
    assert w[3, 17] == np.float32(c[idx[3, 17]]) * s
    # a value exactly between two centroids goes to the lower index
    cc = np.array([-1.0, 1.0] + [5.0] * 14, dtype=np.float32)
    i3, _ = O.quantize_cb4(np.zeros((1, 4), dtype=np.float32), cc, norms=np.array([1.0], dtype=np.float32))
    assert i3[0, 0] == 0
    # a zero row has norm 0 and decodes to zeros
    i4, n4 = O.quantize_cb4(np.zeros((1, 64), dtype=np.float32), c)
    assert n4[0] == 0 and np.all(O.dequant_cb4(O.pack_nibbles(i4), n4, c, 64) == 0)


def _bf16_of_sqrt_by_decimal(row) -> float:
    """Independent check of the codebook norm: sqrt of the exact sum of squares to 120
    decimal digits (exact when the sum is a perfect square), then the nearest bf16 value
    by direct distance among the three candidates around a first guess, ties to the even
    encoding."""
    from decimal import Decimal, getcontext
    from fractions import Fraction
    getcontext().prec = 120
    S = sum((Fraction(float(v)) ** 2 for v in row), Fraction(0))
    if S == 0:
        return 0.0
    root = (Decimal(S.numerator) / Decimal(S.denominator)).sqrt()
    guess = int(O.bf16_bits(O.bf16_from_f64(np.array([float(root)])))[0])
    best = None
    for b in (guess - 1, guess, guess + 1):
        if b < 0 or b > 0x7F7F:
            continue
        v = Decimal(float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0]))
        d = abs(v - root)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return float(np.array([best[1] << 16], dtype=np.uint32).view(np.float32)[0])


def test_cb4_norm_is_exact_bf16_of_row_norm():
    """The codebook norm is the bf16 of the exact Euclidean norm, rounded once: pinned to
    a 120-digit decimal square root on random rows and on rows built to sit exactly on,
    just above and just below a rounding midpoint, where a float64 sum of the squares is
    ambiguous; a permuted row gives the same norm."""
    rng = np.random.default_rng(44)
    rows = [(rng.standard_normal(37) * 0.02).astype(np.float32) for _ in range(6)]
    m = np.float32(1.0 + 3 * 2 ** -8)                 # midpoint of bf16 1+2^-7 and 1+2^-6 ... odd/even pair
    rows.append(np.array([m], dtype=np.float32))      # sqrt(S) == midpoint: tie to even
    rows.append(np.array([m, 2.0 ** -60], dtype=np.float32))    # just above: float64 sum cannot see it
    rows.append(np.array([np.nextafter(m, np.float32(0))], dtype=np.float32))   # just below
    m2 = np.float32(1.0 + 2 ** -8)                    # midpoint of 1 and 1+2^-7
    rows.append(np.array([m2], dtype=np.float32))
    rows.append(np.array([m2, 2.0 ** -70], dtype=np.float32))
    rows.append(np.array([3.0, 4.0] + [0.0] * 5, dtype=np.float32))             # exactly 5
    rows.append(np.array([1e-30, 3e-31], dtype=np.float32))                     # tiny squares
    rows.append(np.array([3e38, 3e38, 3e38, 3e38], dtype=np.float32))           # norm beyond bf16 max
    K = max(len(r) for r in rows)
    w = np.zeros((len(rows), K), dtype=np.float32)
    for i, r in enumerate(rows):
        w[i, :len(r)] = r
    got = O.row_norm_bf16(w)
    for i, r in enumerate(rows[:-1]):
        assert got[i] == _bf16_of_sqrt_by_decimal(r), (i, got[i])
    assert np.isinf(got[-1])
    assert got[6] == np.float32(1.0 + 2 ** -6)        # tie -> even encoding
    assert got[7] == np.float32(1.0 + 2 ** -6) and got[8] == np.float32(1.0 + 2 ** -7)
    assert got[9] == np.float32(1.0) and got[10] == np.float32(1.0 + 2 ** -7)
    assert got[11] == np.float32(5.0)
    perm = rows[0][rng.permutation(len(rows[0]))]
    assert O.row_norm_bf16(perm[None, :])[0] == got[0]


def test_cb4_norm_is_rounded_row_norm():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((4, 300)) * 0.02).astype(np.float32)
    _, n = O.quantize_cb4(w, O.lloyd_max_gaussian()[0])
    for r in range(4):
        exact = math.sqrt(math.fsum(float(v) ** 2 for v in w[r]))
        cands = O.bf16_round(np.array([np.nextafter(np.float32(exact), -np.inf), exact,
                                       np.nextafter(np.float32(exact), np.inf)], dtype=np.float32))
        assert n[r] in cands
        assert abs(n[r] - exact) <= exact * 2 ** -8


def test_storage_accounting_about_25_percent():
    for N, K, approx in [(int(a), int(b), float(c)) for a, b, c in _golden("orbitquant_storage.txt")]:
        b = O.canonical_bytes("cb4", N, K)
        ratio = (b["codes"] + b["scales"] + b["aux"]) / (2 * N * K)
        assert abs(ratio - approx) < 0.001
    b = O.canonical_bytes("cb4", 3072, 3072)
    assert b["codes"] + b["scales"] + b["aux"] == 3072 * 3072 // 2 + 2 * 3072 + 64


# ----------------------------------------------------------------------------- SwiGLU

def test_swiglu_closed_forms():
    up_gate = np.array([[2.0, 0.0, 3.0, 1.0, 5.0, -50.0]], dtype=np.float32)  # up=[2,0,3] gate=[1,5,-50]
    h = O.swiglu_bf16(up_gate)
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    assert h[0, 0] == O.bf16_from_f64(np.array([2 * silu1]))[0] == np.float32(1.4609375)
    assert h[0, 1] == 0.0
    assert abs(h[0, 2]) < 1e-18                       # 3 * silu(-50) ~ 3 * -50 e^-50
    assert O.silu64(np.array([0.0]))[0] == 0.0
    # order of halves: [up | gate], not [gate | up]
    # up=1, gate=2: silu(2) = 2/(1+e^-2) = 1.76159.. -> bf16 1.7578125 (swapped halves: 1.4609375)
    assert O.swiglu_bf16(np.array([[1.0, 2.0]], dtype=np.float32))[0, 0] == np.float32(1.7578125)


# ----------------------------------------------------------------------------- linear

def _frac_linear(a, dw, bias):
    M, K = a.shape
    N = dw.shape[0]
    out = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(a[m, k])) * Fraction(float(dw[n, k]))
            if bias is not None:
                acc += Fraction(float(bias[n]))
            out[m][n] = acc
    return out


@pytest.mark.parametrize("fmt", ["int4_sym", "int4_asym", "mxfp4", "int8", "cb4"])
def test_linear_brute_force_exact_rationals(fmt):
    rng = np.random.default_rng(11)
    M, N, K = 3, 4, 256
    x = S.to_bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = S.to_bf16_values((rng.standard_normal(N) * 0.01).astype(np.float32))
    if fmt == "int4_sym":
        canon = O.quantize("int4", w, 128, symmetric=True)
        f = "int4"
    elif fmt == "int4_asym":
        canon = O.quantize("int4", w, 64, symmetric=False)
        f = "int4"
    elif fmt == "int8":
        canon = O.quantize("int8", w, 128)
        f = "int8"
    else:
        canon = O.quantize(fmt, w)
        f = fmt
    dw = O.dequant(f, canon, K)
    y = O.linear_ref(x, dw, b)
    ex = _frac_linear(x, dw, b)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ex[m][n]) <= abs(ex[m][n]) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
    # dequantised weights stay close to the master weights (catches a wrong scale or sign)
    assert np.max(np.abs(dw - w)) < 0.25 * np.max(np.abs(w))
    # swapping the roles of the operands gives a different, wrongly shaped product
    assert y.shape == (M, N)


def test_grouped_brute_force_exact_rationals():
    """The grouped (MoE) product row by row in exact rational arithmetic: each token's
    row uses its own expert's weights, experts in order, clipped counts."""
    rng = np.random.default_rng(21)
    T, N, K, E = 7, 3, 128, 4
    x = S.to_bf16_values(rng.standard_normal((T, K)).astype(np.float32))
    canons, dws, biases = [], [], []
    for e in range(E):
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        canons.append(O.quantize("mxfp4", w))
        dws.append(O.dequant("mxfp4", canons[-1], K))
        biases.append(S.to_bf16_values((rng.standard_normal(N) * 0.01).astype(np.float32)))
    counts = [2, 0, -3, 9]           # expert 2 counts as empty, expert 3 is clipped to 5 rows
    y = O.forward_grouped("mxfp4", x, canons, counts, K, N, biases)
    owner = [0, 0, 3, 3, 3, 3, 3]
    for t in range(T):
        ex = _frac_linear(x[t:t + 1], dws[owner[t]], biases[owner[t]])[0]
        for n in range(N):
            assert abs(Fraction(y[t, n]) - ex[n]) <= abs(ex[n]) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
    # fewer tokens than rows: the rest stays unset
    y2 = O.forward_grouped("mxfp4", x, canons, [1, 1, 0, 0], K, N)
    assert np.all(np.isnan(y2[2:])) and np.all(np.isfinite(y2[:2]))


def test_output_rows_matches_full_forward():
    rng = np.random.default_rng(12)
    wl = S.small("int8_swiglu", N=64, K=512)
    w = S.weights(wl)
    x = S.activations(wl, 5)
    b = S.bias(wl)
    canon = O.quantize("int8", w, 256)
    y = O.forward("int8", x, canon, 512, b, swiglu=True)
    rows = rng.integers(0, 5, 40)
    cols = rng.integers(0, 64, 40)
    ys = O.output_rows("int8", x, canon, 512, rows, cols, b, swiglu=True)
    assert np.allclose(ys, y[rows, cols], rtol=1e-12, atol=1e-15)


def test_synthetic_workloads_shapes_and_outliers():
    wl = S.small("mxfp4_up", N=200, K=512)
    w = S.weights(wl)
    assert w.shape == (200, 512)
    plain = S.weights(dict(wl, outlier_frac=None))
    changed = w != plain
    assert int(changed.sum()) == round(0.001 * 200 * 512)
    assert np.allclose(w[changed], 20 * plain[changed])
    x = S.activations(S.WORKLOADS["int8_swiglu"], 1, K=64)
    assert x.shape == (1, 128)
    assert np.array_equal(O.bf16_round(x), x)


# ------------------------------------------------- INT8 low-rank merge (addmm_) and its RNG

def test_splitmix64_known_answers():
    rows = {r[0]: r[1:] for r in _golden("splitmix64.txt")}
    seed, *vals = rows["first5"]
    got = O.splitmix64(int(seed), np.arange(5))
    assert [int(v) for v in got] == [int(v) for v in vals]
    seed, *counts = rows["buckets5"]
    z = O.splitmix64(int(seed), np.arange(100000))
    buckets = [(int(v) * 5) >> 64 for v in z]
    assert list(np.bincount(buckets, minlength=5)) == [int(c) for c in counts]


def test_uniform24_is_the_top_bits():
    z = O.splitmix64(99, np.arange(1000))
    u = O.uniform24(99, np.arange(1000))
    assert u.dtype == np.float32
    assert np.all((u >= 0) & (u < 1))
    assert all(Fraction(float(a)) == Fraction(int(b) >> 40, 1 << 24) for a, b in zip(u, z))


def _int8_canon(rng, N, K, G):
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return O.quantize("int8", w, G)


def test_merge_identity_when_alpha_is_zero():
    """beta = 1, alpha = 0 requantises D(W) itself: every RTN group holds a code of
    magnitude 127, so the scale and every code come back unchanged, in both modes."""
    rng = np.random.default_rng(0)
    for G in (32, 64, 256):
        c = _int8_canon(rng, 5, 512, G)
        m1 = S.to_bf16_values(rng.standard_normal((5, 4)).astype(np.float32))
        m2 = S.to_bf16_values(rng.standard_normal((4, 512)).astype(np.float32))
        for seed in (None, 0, 2 ** 64 - 1):
            out = O.merge_lowrank_int8(c, m1, m2, alpha=0.0, beta=1.0, seed=seed)
            assert np.array_equal(out["codes"], c["codes"]) and np.array_equal(out["scales"], c["scales"])


def _exact_fixture(rng, N, K, G, r, beta):
    """Dyadic inputs whose float32 merge is exact and whose new scale is a power of two:
    old scales 2^-5, codes |q| <= 100 except one planted +-127 per group at a k where
    mat2 is zero, mat1 and mat2 in quarter steps.  Then amax = 127 * beta / 32 exactly
    and s' = beta / 32."""
    q = rng.integers(-100, 101, (N, K)).astype(np.int8)
    m2 = (rng.integers(-2, 3, (r, K)) / 4.0).astype(np.float32)
    for g in range(K // G):
        q[:, g * G] = rng.choice([-127, 127], N)
        m2[:, g * G] = 0.0
    m1 = (rng.integers(-2, 3, (N, r)) / 4.0).astype(np.float32)
    scales = O.bf16_bits(np.full((N, K // G), 2.0 ** -5, np.float32))
    return dict(codes=q, scales=scales, group=G), m1, m2


def _brute_merge(canon, m1, m2, alpha, beta, seed):
    """The merge in exact rational arithmetic, codes by exhaustive search over -127..127."""
    q, G = canon["codes"], canon["group"]
    N, K = q.shape
    r = m1.shape[1]
    s_old = Fraction(2) ** -5
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, K // G), np.float64)
    cand = list(range(-127, 128))
    for n in range(N):
        for g in range(K // G):
            ks = range(g * G, (g + 1) * G)
            w = {}
            for k in ks:
                d = sum(Fraction(float(m1[n, j])) * Fraction(float(m2[j, k])) for j in range(r))
                w[k] = Fraction(beta) * int(q[n, k]) * s_old + Fraction(alpha) * d
            amax = max(abs(v) for v in w.values())
            s = amax / 127
            scales[n, g] = float(s)
            for k in ks:
                if seed is None:
                    best = min(abs(w[k] - c * s) for c in cand)
                    ties = [c for c in cand if abs(w[k] - c * s) == best]
                    codes[n, k] = [c for c in ties if c % 2 == 0][0] if len(ties) > 1 else ties[0]
                else:
                    lo = max(c for c in cand if c * s <= w[k])
                    dist = w[k] / s - lo
                    u = Fraction(int(O.splitmix64(seed, n * K + k)) >> 40, 1 << 24)
                    codes[n, k] = min(lo + 1, 127) if u < dist else lo
    return codes, scales


@pytest.mark.parametrize("beta,alpha,seed", [(1.0, 0.25, None), (0.5, -0.125, None), (1.0, 0.25, 7),
                                             (0.5, 0.375, 2 ** 63 + 5)])
def test_merge_against_exact_rationals(beta, alpha, seed):
    rng = np.random.default_rng(int(beta * 8) + (seed or 0) % 97)
    N, K, G, r = 3, 64, 32, 3
    canon, m1, m2 = _exact_fixture(rng, N, K, G, r, beta)
    out = O.merge_lowrank_int8(canon, m1, m2, alpha=alpha, beta=beta, seed=seed)
    codes, scales = _brute_merge(canon, m1, m2, alpha, beta, seed)
    assert np.array_equal(O.bf16_from_bits(out["scales"]).astype(np.float64), scales)
    assert np.array_equal(out["codes"], codes)
    # the fixture must reach rounding ties (nearest) or fractional distances (stochastic)
    if seed is not None:
        assert not np.array_equal(out["codes"], O.merge_lowrank_int8(canon, m1, m2, alpha=alpha, beta=beta)["codes"])


def test_merge_stochastic_is_unbiased_and_picks_neighbours():
    """Over many seeds the mean code is w / s' (the draw is unbiased), every code is one
    of the two neighbours of w / s', and a larger distance means the upper code more
    often."""
    rng = np.random.default_rng(3)
    N, K, G, r = 4, 256, 64, 8
    c = _int8_canon(rng, N, K, G)
    m1 = S.to_bf16_values((rng.standard_normal((N, r)) * 0.05).astype(np.float32))
    m2 = S.to_bf16_values((rng.standard_normal((r, K)) * 0.05).astype(np.float32))
    det = O.merge_lowrank_int8(c, m1, m2, alpha=0.7, beta=0.9)
    s = np.repeat(O.bf16_from_bits(det["scales"]), G, axis=1).astype(np.float64)
    w = 0.9 * O.dequant("int8", c, K).astype(np.float64) + 0.7 * (m1.astype(np.float64) @ m2.astype(np.float64))
    v = w / s
    draws = np.stack([O.merge_lowrank_int8(c, m1, m2, alpha=0.7, beta=0.9, seed=sd)["codes"] for sd in range(300)])
    inside = np.abs(v) <= 127            # beyond +-127 (a group's amax, when bf16 rounded
    assert np.all((draws == np.floor(v)) | (draws == np.floor(v) + 1) | ~inside)   # s' down) clamps
    assert np.all(np.abs(draws[:, ~inside]) == 127)
    mean = draws.astype(np.float64).mean(axis=0)
    assert np.max(np.abs(mean - v)[inside]) < 6 * 0.5 / np.sqrt(300)
    frac = (v - np.floor(v))[inside]
    up = (draws == np.floor(v) + 1).mean(axis=0)[inside]
    assert np.corrcoef(frac, up)[0, 1] > 0.95
    # the scales are the deterministic ones in every draw
    assert all(np.array_equal(O.merge_lowrank_int8(c, m1, m2, 0.7, 0.9, seed=sd)["scales"], det["scales"])
               for sd in (1, 2))


def test_merge_rows_subset_matches_full():
    rng = np.random.default_rng(4)
    c = _int8_canon(rng, 9, 128, 32)
    m1 = S.to_bf16_values(rng.standard_normal((9, 5)).astype(np.float32) * 0.01)
    m2 = S.to_bf16_values(rng.standard_normal((5, 128)).astype(np.float32))
    full = O.merge_lowrank_int8(c, m1, m2, 1.5, 1.0, seed=11)
    rows = np.array([7, 0, 4])
    part = O.merge_lowrank_int8(c, m1, m2, 1.5, 1.0, seed=11, rows=rows)
    assert np.array_equal(part["codes"], full["codes"][rows]) and np.array_equal(part["scales"], full["scales"][rows])


def _rn32(x: Fraction) -> float:
    """Round a rational to the nearest float32 (ties to even), subnormals included."""
    if x == 0:
        return 0.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()      # 2^(e-1) <= a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (max(e, -126) - 23)                           # spacing of float32 at a
    m = a / q
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return float(n * q) if x > 0 else -float(n * q)


def test_lowrank_product_is_a_chain_of_fused_multiply_adds():
    """d_j = fp32(d_{j-1} + a_j b_j) with the exact product, checked against exact rational
    arithmetic and a correct rounding to float32; the operands reach products far below
    the float32 normal range, where a separately rounded product would differ."""
    rng = np.random.default_rng(12)
    R, C, r = 6, 40, 7

    def bf16_vals(shape, lo, hi):
        mant = 1 + rng.integers(0, 128, shape) / 128.0
        ex = rng.integers(lo, hi, shape)
        sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        return (sign * mant * np.exp2(ex)).astype(np.float32)

    m1, m2 = bf16_vals((R, r), -75, 6), bf16_vals((r, C), -75, 6)
    m1[:2] = bf16_vals((2, r), -76, -68)           # products near and below 2^-140, where
    m2[:, :12] = bf16_vals((r, 12), -76, -68)      # float32 is subnormal (spacing 2^-149)
    assert np.array_equal(S.to_bf16_values(m1), m1) and np.array_equal(S.to_bf16_values(m2), m2)
    got = O.lowrank_product_f32(m1, m2)
    for i in range(R):
        for k in range(C):
            d = 0.0
            for j in range(r):
                d = _rn32(Fraction(d) + Fraction(float(m1[i, j])) * Fraction(float(m2[j, k])))
            assert np.float32(d).view(np.uint32) == got[i, k].view(np.uint32), (i, k)
    sep = np.zeros((R, C), np.float32)
    for j in range(r):
        sep = sep + m1[:, j:j + 1] * m2[j:j + 1, :]
    assert not np.array_equal(sep, got)          # the fixture tells the two semantics apart


# ------------------------------------------- INT8-compute path: activation quantisation

def test_activation_quant_on_grid_ties_and_zero_rows():
    rng = np.random.default_rng(20)
    K = 96
    q = rng.integers(-127, 128, (4, K))
    q[:, 5] = 127
    q[1, 9] = -127
    x_grid = (q * 2.0 ** -3).astype(np.float32)                     # s = 2^-3 exactly
    t = rng.integers(-126, 126, (3, K)).astype(np.float64) + 0.5
    t[:, 0] = 127.0
    x_tie = (t * 2.0 ** -4).astype(np.float32)                      # every other value a rint tie
    x = np.vstack([x_grid, x_tie, np.zeros((1, K), np.float32)])
    assert np.array_equal(S.to_bf16_values(x), x)                   # bf16 activations
    codes, s = O.quantize_activations_int8(x)
    assert np.array_equal(s[:4], np.full(4, 0.125, np.float32)) and np.array_equal(codes[:4], q)
    assert np.array_equal(s[4:7], np.full(3, 2.0 ** -4, np.float32))
    lo = np.floor(t)
    even = np.where(lo % 2 == 0, lo, lo + 1)                        # ties to the even code
    assert np.array_equal(codes[4:7], np.where(t == np.rint(t), t, even).astype(np.int8))
    assert s[7] == 0 and not codes[7].any()


def test_activation_quant_error_bound():
    rng = np.random.default_rng(21)
    x = S.to_bf16_values(rng.standard_normal((16, 512)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (16, 1))))
    codes, s = O.quantize_activations_int8(x)
    assert np.array_equal(s, (np.abs(x).max(axis=1) / np.float32(127)).astype(np.float32))
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * s[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 128 * 2.0 ** -23))     # + the rounding of x / s
    assert np.all(np.abs(codes).max(axis=1) == 127)


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("int8", 128)])
def test_forward_a8_exact_rationals(fmt, G):
    rng = np.random.default_rng(22)
    M, N, K = 3, 4, 256
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    canon = O.quantize(fmt, w, G, symmetric=True)
    x = S.to_bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    b = S.to_bf16_values(rng.standard_normal(N).astype(np.float32) * 0.01)
    y = O.forward_a8(fmt, x, canon, K, b)
    codes, s = O.quantize_activations_int8(x)
    dw = O.dequant(fmt, canon, K)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(int(codes[m, k])) * Fraction(float(s[m])) * Fraction(float(dw[n, k]))
                        for k in range(K)) + Fraction(float(b[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
