"""On-device round-to-nearest quantiser against the oracle's quantisers: byte for byte.

The quantiser has a unique answer under the rounding rules (round to nearest even at
every float32 operation, ties of rint to even, E2M1 ties to the even code, codebook
ties to the lower index), so every code, scale and zero-point must equal the oracle's.
Inputs mix Gaussian weights, outliers, all-zero groups, tiny (subnormal-range) groups,
values on the grid and values exactly half-way between grid points (rounding ties).
The quantised weights then go through pack and the forward kernel and must meet the
usual tolerance against the oracle's linear.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import rel_err, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _lib():
    import bit_weight_only_offline_amd as Q
    return Q


def _weights(fmt, N, K, G, seed):
    """Gaussian weights with planted special groups (each a whole group of one row)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[rng.random((N, K)) < 0.002] *= 20.0                     # outliers
    g = 32 if fmt in ("mxfp4", "cb4") else G
    ng = K // g
    specials = []
    # all-zero group, tiny group (amax in the float32 subnormal range), huge-ish group
    specials.append(np.zeros(g, np.float32))
    specials.append((rng.standard_normal(g) * 1e-41).astype(np.float32))
    specials.append((rng.standard_normal(g) * 3.0).astype(np.float32))
    if fmt == "int4":
        s = np.float32(np.float16(0.01))                       # an fp16 step
        q = rng.integers(-7, 8, g).astype(np.float32)
        q[0] = 7.0
        specials.append(q * s)                                 # on the symmetric grid
        t = (rng.integers(-6, 6, g) + 0.5).astype(np.float32)
        t[0] = 7.0
        specials.append(t * s)                                 # rint ties (x.5 steps)
    elif fmt == "int8":
        s = np.float32(O.bf16_round(np.float32(0.002)))
        q = rng.integers(-127, 128, g).astype(np.float32)
        q[0] = 127.0
        specials.append(q * s)
        t = (rng.integers(-120, 120, g) + 0.5).astype(np.float32)
        t[0] = 127.0
        specials.append(t * s)
    elif fmt == "mxfp4":
        mags = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6], np.float32)
        v = rng.choice(mags, g) * np.where(rng.random(g) < 0.5, -1, 1).astype(np.float32)
        v[0] = 6.0
        specials.append(v * np.float32(2.0 ** -5))           # every E2M1 tie, amax = 6 * 2^e
        v2 = v.copy()
        v2[0] = -0.0
        v2[1] = 4.0
        specials.append(v2 * np.float32(2.0 ** 3))
    rows = rng.choice(N, size=min(N, len(specials)), replace=False)
    for r, sp in zip(rows, specials):
        if fmt == "cb4":
            w[r, :] = np.resize(sp, K)                        # codebook: whole rows
        else:
            j = int(rng.integers(0, ng))
            w[r, j * g:(j + 1) * g] = sp
    return w


CASES = [
    ("int4", 128, True), ("int4", 128, False), ("int4", 32, False), ("int4", 64, True), ("int4", 256, False),
    ("int8", 256, True), ("int8", 64, True), ("int8", 32, True),
    ("mxfp4", 32, True),
    ("cb4", 0, True),
]


def _oracle(fmt, w, G, sym):
    if fmt == "cb4":
        return O.quantize("cb4", w, centroids=O.lloyd_max_gaussian()[0])
    return O.quantize(fmt, w, G, symmetric=sym)


def _device(fmt, w, G, sym):
    Q = _lib()
    lv = O.lloyd_max_gaussian()[0].astype(np.float32) if fmt == "cb4" else None
    return Q.quantize(fmt, torch.from_numpy(w).cuda(), G, symmetric=sym, levels=lv)


@pytest.mark.parametrize("fmt,G,sym", CASES, ids=[f"{c[0]}_g{c[1]}_{'sym' if c[2] else 'asym'}" for c in CASES])
@pytest.mark.parametrize("N,K", [(37, 512), (8, 1536)])
def test_quantize_matches_oracle_bit_exact(fmt, G, sym, N, K):
    w = _weights(fmt, N, K, G, seed=N * 7 + K)
    canon = _oracle(fmt, w, G, sym)
    codes, scales, aux = _device(fmt, w, G, sym)
    torch.cuda.synchronize()
    c_ref, s_ref, _ = to_device(fmt, canon)
    assert torch.equal(codes.cpu(), c_ref.cpu()), "codes"
    assert torch.equal(scales.cpu().view(torch.uint8), s_ref.cpu().view(torch.uint8)), "scales"
    if fmt == "int4" and not sym:
        assert torch.equal(aux.cpu(), torch.from_numpy(canon["zeros"])), "zero-points"


@pytest.mark.parametrize("fmt,G,sym", [("int4", 128, False), ("mxfp4", 32, True), ("int8", 256, True),
                                       ("cb4", 0, True)])
def test_quantize_then_pack_then_forward(fmt, G, sym):
    """Device quantiser -> pack -> linear, against the oracle's quantise -> linear.

    The planted row 150x larger than the rest dominates rms(Y).  For the codebook the
    single bf16 rounding of each level (relative error about 1e-3) would then reach the
    1e-2 gate; the packer sees the spread of the row norms and selects the two-term
    operand, which the record's split flag shows."""
    Q = _lib()
    N, K, M = 96, 1024, 24
    w = _weights(fmt, N, K, G, seed=5)
    canon = _oracle(fmt, w, G, sym)
    codes, scales, aux = _device(fmt, w, G, sym)
    pw = Q.pack(fmt, N, K, G, codes, scales, aux)
    if fmt == "cb4":
        assert int(pw.aux.cpu().numpy()[104:108].view(np.uint32)[0]) == 1
    x = S.to_bf16_values(np.random.default_rng(3).standard_normal((M, K)).astype(np.float32))
    y = Q.linear(torch.from_numpy(x).cuda().to(torch.bfloat16), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref = O.forward(fmt, x, canon, K)
    assert rel_err(y.cpu().numpy(), yref) <= 1e-2


@pytest.mark.parametrize("name", ["int4_asym_decode", "mxfp4_down", "cb4_prefill"])
def test_quantize_full_size_workload(name):
    """The workload's own weights at full size: bit-exact with the oracle."""
    wl = S.WORKLOADS[name]
    fmt, G, sym = wl["fmt"], wl["group"], wl.get("symmetric", True)
    print(f"quantize {name} N={wl['N']} K={wl['K']}", flush=True)
    w = S.weights(wl)
    canon = _oracle(fmt, w, G, sym)
    codes, scales, aux = _device(fmt, w, G, sym)
    torch.cuda.synchronize()
    c_ref, s_ref, _ = to_device(fmt, canon)
    assert torch.equal(codes, c_ref)
    assert torch.equal(scales.view(torch.uint8), s_ref.view(torch.uint8))
    if fmt == "int4" and not sym:
        assert torch.equal(aux.cpu(), torch.from_numpy(canon["zeros"]))


def test_codebook_norm_exact_at_rounding_midpoints():
    """Rows whose exact norm sits on, just above and just below a bf16 rounding midpoint
    (where any float64 sum of the squares is ambiguous), rows spanning the float32
    exponent range, the overflow and the all-zero row: the device norm is the oracle's
    bf16 of the exact norm, bit for bit (both sum the squares exactly)."""
    rng = np.random.default_rng(71)
    K = 64
    rows = []
    for k in range(48):
        mant = int(rng.integers(256, 512))
        m = np.float32(np.ldexp(float(2 * mant + 1), int(rng.integers(-60, 60)) - 9))
        r = np.zeros(K, np.float32)
        r[int(rng.integers(0, K))] = m
        if k % 3 == 1:
            r[(int(rng.integers(0, K)) + 1) % K] = np.float32(np.ldexp(1.0, -50) * abs(float(m)))
        if k % 3 == 2:
            r[r != 0] = np.nextafter(m, np.float32(0))
        rows.append(r)
    for _ in range(16):
        rows.append((rng.standard_normal(K) * 10.0 ** rng.uniform(-40, 37)).astype(np.float32))
    rows.append(np.array([3e38] * 4 + [0] * (K - 4), np.float32))
    rows.append(np.zeros(K, np.float32))
    w = np.stack(rows)
    canon = _oracle("cb4", w, 0, True)
    codes, scales, _ = _device("cb4", w, 0, True)
    torch.cuda.synchronize()
    c_ref, s_ref, _ = to_device("cb4", canon)
    assert torch.equal(scales.cpu().view(torch.uint8), s_ref.cpu().view(torch.uint8)), "norms"
    assert torch.equal(codes.cpu(), c_ref.cpu()), "codes"
