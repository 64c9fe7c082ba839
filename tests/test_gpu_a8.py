"""INT8-compute linear (W4A8 / W8A8) through the C ABI against the oracle.

The activation quantiser has a unique answer (float32, RNE, ties to even), so its codes
and scales must equal the oracle's byte for byte.  The linear sums exact int32 products
per weight group and applies the group and row scales in float32, so against the oracle's
exact product of the same quantised activations (forward_a8) the only error is float32
rounding of the group folding: G2 is checked at the usual 1e-2 and at a tight 1e-5, and
the bf16 output must be the RNE rounding of the float32 one (G3).
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import rel_err, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _x(rng, M, K, special=True):
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp2(rng.integers(-6, 6, (M, 1))).astype(np.float32)        # rows of different scale
    if special and M >= 4:
        x[1] = 0.0                                                         # all-zero row
        t = (rng.integers(-126, 126, K) + 0.5).astype(np.float32)
        t[0] = 127.0
        x[2] = t * np.float32(2.0 ** -5)                                   # rint ties (x.5 steps)
        x[3, :] *= np.float32(1e-30)                                       # tiny row
    return S.to_bf16_values(x)


@pytest.mark.parametrize("M,K", [(1, 96), (37, 512), (130, 4096), (4, 28672)])
def test_activation_quant_bit_exact(M, K):
    import bit_weight_only_offline_amd as Q
    x = _x(np.random.default_rng(M + K), M, K)
    codes, scales = Q.quantize_activations(torch.from_numpy(x).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    c_ref, s_ref = O.quantize_activations_int8(x)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


CASES = [("int4", 64), ("int4", 128), ("int4", 256), ("int8", 64), ("int8", 128), ("int8", 256)]


@pytest.mark.parametrize("fmt,G", CASES, ids=[f"{f}_g{g}" for f, g in CASES])
@pytest.mark.parametrize("M", [1, 5, 16, 17, 40, 64, 65, 150])
def test_linear_a8_matches_oracle(fmt, G, M):
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(M * 7 + G)
    N, K = 200, 768
    canon = O.quantize(fmt, (rng.standard_normal((N, K)) * 0.02).astype(np.float32), G, symmetric=True)
    pw = Q.pack(fmt, N, K, G, *to_device(fmt, canon))
    x = _x(rng, M, K)
    b = S.to_bf16_values((rng.standard_normal(N) * 0.01).astype(np.float32))
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    bt = torch.from_numpy(b).cuda().to(torch.bfloat16)
    yref = O.forward_a8(fmt, x, canon, K, b)
    for tile in range(len(Q.a8_tile_shapes())):
        print(f"a8 {fmt} g{G} M={M} tile={tile}", flush=True)
        y32 = Q.linear_a8(xt, pw, bias=bt, out_dtype=torch.float32, tile=tile)
        y16 = Q.linear_a8(xt, pw, bias=bt, tile=tile)
        torch.cuda.synchronize()
        err = rel_err(y32.cpu().numpy(), yref)
        assert err <= 1e-5, (tile, err)
        assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


def test_linear_a8_ragged_and_no_bias():
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(3)
    for fmt, N, K, G in [("int4", 37, 96 * 2, 64), ("int8", 50, 320, 64), ("int4", 21, 1280, 128)]:
        canon = O.quantize(fmt, (rng.standard_normal((N, K)) * 0.02).astype(np.float32), G, symmetric=True)
        pw = Q.pack(fmt, N, K, G, *to_device(fmt, canon))
        x = _x(rng, 23, K)
        y = Q.linear_a8(torch.from_numpy(x).cuda().to(torch.bfloat16), pw, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), O.forward_a8(fmt, x, canon, K)) <= 1e-5, (fmt, N, K)


def test_linear_a8_full_size_prefill_sampled():
    """INT4 g128 3072 x 3072 at M = 2048 (the prefill shape) with the default schedule:
    sampled outputs one by one against the oracle; finite and run-to-run equal."""
    import bit_weight_only_offline_amd as Q
    wl = S.WORKLOADS["cb4_prefill"]
    N, K, M, G = wl["N"], wl["K"], 2048, 128
    rng = np.random.default_rng(5)
    canon = O.quantize("int4", S.weights(wl), G, symmetric=True)
    pw = Q.pack("int4", N, K, G, *to_device("int4", canon))
    x = S.activations(wl, M)
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    print(f"a8 int4 full size M={M} N={N} K={K}", flush=True)
    y1 = Q.linear_a8(xt, pw, out_dtype=torch.float32)
    y2 = Q.linear_a8(xt, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and bool(torch.isfinite(y1).all())
    rows = np.unique(np.concatenate([[0, 1, M - 1], rng.integers(0, M, 8)]))
    cols = np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 8)]))
    q, s = O.quantize_activations_int8(x[rows])
    dw = O.dequant("int4", {k: (v[cols] if isinstance(v, np.ndarray) else v) for k, v in canon.items()}, K)
    ref = (q.astype(np.float64) * s.astype(np.float64)[:, None]) @ dw.astype(np.float64).T
    got = y1.cpu().numpy()[np.ix_(rows, cols)]
    assert np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)) <= 1e-5
