"""Parity at the largest shapes the boundary accepts.

The kernels address activations and packed weights with 32-bit buffer offsets, in
which bit 31 of an activation offset marks a load as out of range (it then reads as
zero).  Validation keeps M * (row length) below 2^30 elements and the packed weight
below 4 GiB.  These tests run right at those limits:

* activations of nearly 2 GiB with an input dimension that is not a multiple of the
  128-wide chunk, in the codebook format, whose padding code decodes to a nonzero
  level: the past-K inputs of the last rows must still read as zero;
* an INT8 weight of nearly 4 GiB, at decode and tile sizes of M.

Inputs are drawn on the device from seeded generators; the oracle computes sampled
outputs (first, last and random rows and columns) one by one from the same values,
copied back to the host.  One size past each limit is refused before any launch.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import bf16_tensor, quantize, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-2


def _lib():
    import bit_weight_only_offline_amd as Q
    return Q


def _check_sample(fmt, y32, y16, x_rows, rows, cols, canon_cols, K, bias_cols=None):
    """G2 on sampled outputs (oracle on the sampled rows and columns), G3 on the whole output."""
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), "G3"
    ref = O.forward(fmt, x_rows, canon_cols, K, bias_cols)           # [len(rows), len(cols)]
    got = y32[torch.as_tensor(rows, device=y32.device)][:, torch.as_tensor(cols, device=y32.device)]
    got = got.cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) / rms
    print(f"  sampled {ref.size} outputs: max|dY|/rms = {err:.3e}", flush=True)
    assert err <= TOL


def test_largest_activation_ragged_k_codebook():
    """M * K just below 2^30 with K = 160 (the last chunk runs 96 inputs past K): the
    last row's past-K inputs lie within 2 * 128 bytes of the 2 GiB offset limit."""
    Q = _lib()
    N, K = 24, 160
    M = ((1 << 30) - 1) // K                       # 6710886 rows, M * K = 2^30 - 64
    print(f"limits: codebook N={N} K={K} M={M}", flush=True)
    rng = np.random.default_rng(41)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    canon = quantize("cb4", w, 0)
    codes, scales, aux = to_device("cb4", canon)
    pw = Q.pack("cb4", N, K, 0, codes, scales, aux)
    b = S.to_bf16_values((rng.standard_normal(N) * 0.01).astype(np.float32))
    bias = bf16_tensor(b)
    g = torch.Generator(device="cuda").manual_seed(41)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)

    y32 = Q.linear(x, pw, bias, out_dtype=torch.float32)
    y16 = Q.linear(x, pw, bias)
    torch.cuda.synchronize()
    assert torch.isfinite(y32).all()

    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 3, M - 2, M - 1], rng.integers(0, M, 10)]))
    cols = np.arange(N)
    x_rows = x[torch.as_tensor(rows, device="cuda")].float().cpu().numpy()
    _check_sample("cb4", y32, y16, x_rows, rows, cols, canon, K, b)

    # one row more crosses the limit: refused before any launch
    x1 = torch.zeros((M + 1, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Q.QLinearError):
        Q.linear(x1, pw)


def test_largest_int8_weight():
    """An INT8 weight of N x K = 1048560 x 4096 bytes, 64 KiB below 4 GiB, whose last
    column tile ends 64 KiB before the 32-bit offset limit."""
    Q = _lib()
    K, G = 4096, 256
    N = (1 << 32) // K - 16
    print(f"limits: int8 N={N} K={K}", flush=True)
    wb, sb, _ = Q.packed_bytes("int8", N, K, G)
    assert wb < (1 << 32) <= wb + 16 * K
    g = torch.Generator(device="cuda").manual_seed(42)
    codes = torch.randint(-127, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
    sc = (torch.rand((N, K // G), generator=g, device="cuda") * 0.02 + 1e-3).to(torch.bfloat16)
    pw = Q.pack("int8", N, K, G, codes, sc)

    rng = np.random.default_rng(42)
    cols = np.unique(np.concatenate([[0, 1, N // 2, N - 17, N - 2, N - 1], rng.integers(0, N, 58)]))
    cidx = torch.as_tensor(cols, device="cuda")
    canon_cols = {"codes": codes[cidx].cpu().numpy(), "group": G,
                  "scales": sc[cidx].view(torch.int16).cpu().numpy().view(np.uint16)}
    del codes
    torch.cuda.synchronize()
    for M in (1, 16, 64):
        x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
        print(f"  M={M} schedule={Q.default_schedule('int8', M, N, K, G)}", flush=True)
        y32 = Q.linear(x, pw, out_dtype=torch.float32)
        y16 = Q.linear(x, pw)
        torch.cuda.synchronize()
        assert torch.isfinite(y32).all()
        rows = np.arange(M) if M <= 16 else np.unique(np.concatenate([[0, 1, M - 1], rng.integers(0, M, 8)]))
        x_rows = x[torch.as_tensor(rows, device="cuda")].float().cpu().numpy()
        y32s = y32[:, cidx].contiguous()
        y16s = y16[:, cidx].contiguous()
        _check_sample("int8", y32s, y16s, x_rows, rows, np.arange(len(cols)), canon_cols, K)

    # a weight one column tile larger does not fit 32-bit offsets: refused
    with pytest.raises(Q.QLinearError):
        Q.packed_bytes("int8", N + 16, K, G)


def test_grouped_many_experts_past_decode_grid():
    """70000 experts with one token each: the ceil(T/16) + E slots of the decode kernel
    exceed the grid's second dimension (65535), so the 32-row ring tile serves, with its
    slots along the first.  Sampled tokens against the oracle, each with its own expert."""
    Q = _lib()
    E = T = 70000
    N, K, G = 16, 128, 128
    print(f"limits: grouped int4 E={E} T={T} N={N} K={K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(43)
    codes = torch.randint(0, 256, (E * N, K // 2), generator=g, device="cuda", dtype=torch.uint8)
    scales = (torch.rand((E * N, K // G), generator=g, device="cuda") * 0.02 + 1e-3).to(torch.float16)
    pe = Q.pack_experts("int4", N, K, G, [(codes[e * N:(e + 1) * N], scales[e * N:(e + 1) * N], None)
                                          for e in range(E)])
    x = torch.randn((T, K), generator=g, device="cuda", dtype=torch.bfloat16)
    counts = torch.ones(E, dtype=torch.int32, device="cuda")
    y32 = Q.grouped_linear(x, pe, counts, out_dtype=torch.float32)
    y16 = Q.grouped_linear(x, pe, counts)
    torch.cuda.synchronize()
    assert torch.isfinite(y32).all()
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), "G3"

    rng = np.random.default_rng(43)
    tokens = np.unique(np.concatenate([[0, 1, T // 2, T - 2, T - 1], rng.integers(0, T, 20)]))
    refs, gots = [], []
    for t in tokens:
        canon = {"codes": codes[t * N:(t + 1) * N].cpu().numpy(), "scales": scales[t * N:(t + 1) * N].cpu().numpy(),
                 "zeros": None, "group": G}
        refs.append(O.forward("int4", x[t:t + 1].float().cpu().numpy(), canon, K)[0])
        gots.append(y32[t].cpu().numpy().astype(np.float64))
    ref, got = np.array(refs), np.array(gots)
    err = float(np.max(np.abs(got - ref))) / float(np.sqrt(np.mean(ref ** 2)))
    print(f"  sampled {ref.size} outputs: max|dY|/rms = {err:.3e}", flush=True)
    assert err <= TOL
