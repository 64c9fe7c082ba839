"""Grouped (mixture-of-experts) linear through the C ABI against the oracle.

Tokens are grouped by expert in expert order; each row must match the oracle's product
with its own expert's weights (G2), the bf16 output is the RNE rounding of the float32
one (G3), each expert's rows equal the dense kernel with the same tile schedule run on
that expert alone (bit for bit), rows past the sum of the counts are left untouched,
and counts are clipped as documented (negative -> 0, nothing past T).
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import quantize, rel_err, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-2
FORMATS = [("int4", 128, False), ("int4", 64, True), ("mxfp4", 32, True), ("int8", 256, True), ("cb4", 0, True)]


def _experts(fmt, G, sym, E, N, K, seed):
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(seed)
    canons, dev = [], []
    for _ in range(E):
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        canon = quantize(fmt, w, G, sym)
        canons.append(canon)
        dev.append(to_device(fmt, canon))
    pe = Q.pack_experts(fmt, N, K, G, dev)
    return pe, canons, dev


def _grouped_schedule(Q, T, E, fmt, N, K, G):
    """(tile, rows per slot) the library plans for a grouped call: the decode kernel in
    slots of 16 rows when experts average at most 16 tokens (its four-wavefront
    single-tile schedule, 24, where the dense default is the eight-wavefront one, 0),
    else ring tiles."""
    per = (T + E - 1) // E
    if per <= 16:
        tile = Q.default_schedule(fmt, 16, N, K, G).tile
        return (24 if tile == 0 else tile), 16
    if per <= 48:
        return (17 if fmt in ("int4", "int8") else 5), 32
    if per <= 96:
        return 16, 64
    return (8 if fmt in ("int4", "int8") else 13), 128


@pytest.mark.parametrize("fmt,G,sym", FORMATS, ids=[f"{f}_g{g}_{'sym' if s else 'asym'}" for f, g, s in FORMATS])
@pytest.mark.parametrize("counts", [[3, 0, 70, 1, 40], [130, 2, 0, 200], [0, 0, 5], [20, 0, 1, 1, 2, 0, 0, 0]],
                         ids=["mixed", "large", "one", "decode"])
def test_grouped_matches_oracle_and_dense(fmt, G, sym, counts):
    import bit_weight_only_offline_amd as Q
    E, N, K = len(counts), 200, 512
    T = sum(counts)
    print(f"grouped {fmt} counts={counts} N={N} K={K}", flush=True)
    pe, canons, dev = _experts(fmt, G, sym, E, N, K, seed=T + E)
    rng = np.random.default_rng(T)
    x = S.to_bf16_values(rng.standard_normal((T, K)).astype(np.float32))
    b = S.to_bf16_values((rng.standard_normal((E, N)) * 0.01).astype(np.float32))
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    bt = torch.from_numpy(b).cuda().to(torch.bfloat16)
    cnt = torch.tensor(counts, dtype=torch.int32, device="cuda")
    y32 = Q.grouped_linear(xt, pe, cnt, bias=bt, out_dtype=torch.float32)
    y16 = Q.grouped_linear(xt, pe, cnt, bias=bt)
    torch.cuda.synchronize()
    yref = O.forward_grouped(fmt, x, canons, counts, K, N, list(b))
    assert rel_err(y32.cpu().numpy(), yref) <= TOL
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    # each expert's rows: the dense kernel with the same schedule on that expert alone
    # (the decode kernel slot by slot of 16 rows)
    tile, rows = _grouped_schedule(Q, T, E, fmt, N, K, G)
    step = 16 if rows == 16 else max(counts) + 1
    run = 0
    for e, c in enumerate(counts):
        if c:
            pw = Q.pack(fmt, N, K, G, *dev[e])
            for r in range(0, c, step):
                rr = min(step, c - r)
                yd = Q.linear(xt[run + r:run + r + rr], pw, bias=bt[e], out_dtype=torch.float32, schedule=(tile, 1))
                torch.cuda.synchronize()
                assert torch.equal(yd, y32[run + r:run + r + rr]), f"expert {e} rows {r}"
        run += c


def test_grouped_clipping_and_untouched_rows():
    import bit_weight_only_offline_amd as Q
    fmt, G, N, K = "mxfp4", 32, 64, 256
    pe, canons, _ = _experts(fmt, G, True, 3, N, K, seed=7)
    T = 20
    x = S.to_bf16_values(np.random.default_rng(1).standard_normal((T, K)).astype(np.float32))
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    for counts in ([5, -4, 9], [12, 0, 50], [0, 0, 0]):
        out = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        cnt = torch.tensor(counts, dtype=torch.int32, device="cuda")
        Q.grouped_linear(xt, pe, cnt, out_dtype=torch.float32, out=out)
        torch.cuda.synchronize()
        yref = O.forward_grouped(fmt, x, canons, counts, K, N)
        y = out.cpu().numpy()
        done = np.isfinite(yref[:, 0])
        assert np.array_equal(np.isnan(y[:, 0]), ~done), counts          # untouched rows stay NaN
        if done.any():
            assert rel_err(y[done], yref[done]) <= TOL


def test_grouped_moe_down_projection_sampled():
    """Eight MXFP4 experts of the down projection (4096 x 14336), 256 routed tokens."""
    import bit_weight_only_offline_amd as Q
    E, N, K, T = 8, 4096, 14336, 256
    rng = np.random.default_rng(8)
    counts = list(np.bincount(rng.integers(0, E, T), minlength=E).astype(int))
    print(f"moe down projection counts={counts}", flush=True)
    pe, canons, _ = _experts("mxfp4", 32, True, E, N, K, seed=9)
    x = S.to_bf16_values(rng.standard_normal((T, K)).astype(np.float32))
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    y = Q.grouped_linear(xt, pe, torch.tensor(counts, dtype=torch.int32, device="cuda"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 30)]))
    run, errs, refs = 0, [], []
    for e, c in enumerate(counts):
        if c:
            rows = np.unique(np.concatenate([[run, run + c - 1], rng.integers(run, run + c, 2)]))
            rr, cc = np.meshgrid(rows - run, cols, indexing="ij")
            ref = O.output_rows("mxfp4", x[run:run + c], canons[e], K, rr.ravel(), cc.ravel())
            refs.append(ref)
            errs.append(np.abs(y[rows][:, cols].ravel() - ref))
        run += c
    ref = np.concatenate(refs)
    err = np.max(np.concatenate(errs)) / np.sqrt(np.mean(ref ** 2))
    print(f"  sampled {ref.size} outputs: max|dY|/rms = {err:.3e}", flush=True)
    assert err <= TOL


def test_grouped_many_experts():
    """More experts than the plan kernel takes in one batch (300 > 256), most of them
    empty or with a few tokens, and counts that run past T."""
    import bit_weight_only_offline_amd as Q
    fmt, G, N, K, E, T = "mxfp4", 32, 32, 128, 300, 180
    rng = np.random.default_rng(30)
    counts = np.where(rng.random(E) < 0.6, 0, rng.integers(1, 4, E)).astype(int)
    counts[-1] = 50                                        # the running sum passes T here
    pe, canons, _ = _experts(fmt, G, True, E, N, K, seed=31)
    x = S.to_bf16_values(rng.standard_normal((T, K)).astype(np.float32))
    xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
    out = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    Q.grouped_linear(xt, pe, torch.tensor(counts, dtype=torch.int32, device="cuda"), out_dtype=torch.float32,
                     out=out)
    torch.cuda.synchronize()
    yref = O.forward_grouped(fmt, x, canons, list(counts), K, N)
    y = out.cpu().numpy()
    done = np.isfinite(yref[:, 0])
    assert np.array_equal(np.isnan(y[:, 0]), ~done)
    assert rel_err(y[done], yref[done]) <= TOL
