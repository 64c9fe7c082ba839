"""In-place INT8 low-rank merge (addmm_) through the C ABI against the oracle: byte for byte.

The merge has a unique answer under its arithmetic (float32, one rounding per operation,
the low-rank product as fused multiply-adds in index order, RTN scales, nearest or
SplitMix64-driven stochastic codes),
so after the update the weight's canonical codes and scales must equal the oracle's, and
the packed buffers must equal the packing of the oracle's result byte for byte (padding
included).  Shapes span several column tiles with a ragged last tile (N not a multiple of
16), several 256-input blocks with a ragged last one, every group size and ranks that are
and are not multiples of the register chunk.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _case(N, K, G, r, seed):
    rng = np.random.default_rng(seed)
    canon = O.quantize("int8", (rng.standard_normal((N, K)) * 0.02).astype(np.float32), G)
    m1 = S.to_bf16_values((rng.standard_normal((N, r)) * 0.05).astype(np.float32))
    m2 = S.to_bf16_values((rng.standard_normal((r, K)) * 0.05).astype(np.float32))
    return canon, m1, m2


def _packed(Q, canon, N, K, G):
    return Q.pack("int8", N, K, G, *to_device("int8", canon))


def _check_equal(Q, pw, ref, N, K, G):
    codes, scales, _ = Q.unpack(pw)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), ref["codes"]), "codes"
    assert np.array_equal(scales.cpu().view(torch.int16).numpy().view(np.uint16), ref["scales"]), "scales"
    want = _packed(Q, ref, N, K, G)
    torch.cuda.synchronize()
    assert torch.equal(pw.w, want.w) and torch.equal(pw.s, want.s), "packed bytes (padding included)"


CASES = [
    # N, K, G, r
    (37, 512, 32, 7), (37, 512, 64, 16), (50, 768, 128, 1), (21, 1024, 256, 33),
    (16, 96, 32, 8), (200, 1536, 256, 64), (40, 640, 64, 100), (19, 256, 256, 256),
]


@pytest.mark.parametrize("N,K,G,r", CASES, ids=[f"N{c[0]}_K{c[1]}_g{c[2]}_r{c[3]}" for c in CASES])
@pytest.mark.parametrize("seed", [None, 0, 12345678901234567890], ids=["nearest", "seed0", "seed_big"])
def test_merge_matches_oracle(N, K, G, r, seed):
    import bit_weight_only_offline_amd as Q
    print(f"int8 merge N={N} K={K} G={G} r={r} seed={seed}", flush=True)
    canon, m1, m2 = _case(N, K, G, r, N * K + r)
    pw = _packed(Q, canon, N, K, G)
    w_ptr, s_ptr = pw.w.data_ptr(), pw.s.data_ptr()
    Q.int8_addmm_(pw, torch.from_numpy(m1).cuda().to(torch.bfloat16), torch.from_numpy(m2).cuda().to(torch.bfloat16),
                  alpha=0.8, beta=1.0, rounding_seed=seed)
    assert pw.w.data_ptr() == w_ptr and pw.s.data_ptr() == s_ptr          # the same storage
    _check_equal(Q, pw, O.merge_lowrank_int8(canon, m1, m2, 0.8, 1.0, seed=seed), N, K, G)


@pytest.mark.parametrize("alpha,beta", [(0.0, 1.0), (1.0, 0.0), (-2.5, 0.75), (3.0, -1.0)])
def test_merge_alpha_beta(alpha, beta):
    import bit_weight_only_offline_amd as Q
    N, K, G, r = 45, 512, 128, 12
    canon, m1, m2 = _case(N, K, G, r, 5)
    for seed in (None, 99):
        pw = _packed(Q, canon, N, K, G)
        Q.int8_addmm_(pw, torch.from_numpy(m1).cuda().to(torch.bfloat16),
                      torch.from_numpy(m2).cuda().to(torch.bfloat16), alpha=alpha, beta=beta, rounding_seed=seed)
        ref = O.merge_lowrank_int8(canon, m1, m2, alpha, beta, seed=seed)
        _check_equal(Q, pw, ref, N, K, G)
        if alpha == 0.0 and beta == 1.0:
            assert np.array_equal(ref["codes"], canon["codes"])              # requantising D(W) is the identity


def test_merge_rank_zero_and_repeated_updates():
    import bit_weight_only_offline_amd as Q
    N, K, G = 33, 512, 64
    canon, m1, m2 = _case(N, K, G, 9, 6)
    pw = _packed(Q, canon, N, K, G)
    e1 = torch.empty((N, 0), dtype=torch.bfloat16, device="cuda")
    e2 = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    Q.int8_addmm_(pw, e1, e2, alpha=1.0, beta=0.5)                      # rank 0: 0.5 W, requantised
    ref = O.merge_lowrank_int8(canon, np.zeros((N, 0), np.float32), np.zeros((0, K), np.float32), 1.0, 0.5)
    _check_equal(Q, pw, ref, N, K, G)
    # a second and a third update on top (each one requantises: the oracle does the same)
    a = torch.from_numpy(m1).cuda().to(torch.bfloat16)
    b = torch.from_numpy(m2).cuda().to(torch.bfloat16)
    Q.int8_addmm_(pw, a, b, alpha=0.5, rounding_seed=3)
    Q.int8_addmm_(pw, a, b, alpha=-0.25)
    ref = O.merge_lowrank_int8(ref, m1, m2, 0.5, 1.0, seed=3)
    ref = O.merge_lowrank_int8(ref, m1, m2, -0.25, 1.0)
    _check_equal(Q, pw, ref, N, K, G)


def test_merge_seed_reproducible_and_distinct():
    import bit_weight_only_offline_amd as Q
    N, K, G, r = 64, 1024, 256, 16
    canon, m1, m2 = _case(N, K, G, r, 8)
    a = torch.from_numpy(m1).cuda().to(torch.bfloat16)
    b = torch.from_numpy(m2).cuda().to(torch.bfloat16)
    outs = []
    for seed in (5, 5, 6):
        pw = _packed(Q, canon, N, K, G)
        Q.int8_addmm_(pw, a, b, alpha=1.0, rounding_seed=seed)
        outs.append(pw.w.clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and not torch.equal(outs[0], outs[2])


def test_merge_full_size_workload_sampled_rows():
    """The INT8 SwiGLU layer's weight (8192 x 28672, group 256) with a rank-16 adapter,
    stochastic: rows sampled across the matrix (first and last included) byte for byte,
    and a second run with the same seed identical over the whole buffer."""
    import bit_weight_only_offline_amd as Q
    wl = S.WORKLOADS["int8_swiglu"]
    N, K, G, r = wl["N"], wl["K"], wl["group"], 16
    rng = np.random.default_rng(21)
    codes, scales, _ = S.random_codes(rng, "int8", N, K, G)
    canon = dict(codes=codes, scales=scales, group=G)
    m1 = S.to_bf16_values((rng.standard_normal((N, r)) * 0.01).astype(np.float32))
    m2 = S.to_bf16_values((rng.standard_normal((r, K)) * 0.01).astype(np.float32))
    print(f"int8 merge full size N={N} K={K} r={r}", flush=True)
    a = torch.from_numpy(m1).cuda().to(torch.bfloat16)
    b = torch.from_numpy(m2).cuda().to(torch.bfloat16)
    pws = []
    for _ in range(2):
        pw = _packed(Q, canon, N, K, G)
        Q.int8_addmm_(pw, a, b, alpha=2.0, beta=1.0, rounding_seed=2 ** 40 + 1)
        pws.append(pw)
    torch.cuda.synchronize()
    assert torch.equal(pws[0].w, pws[1].w) and torch.equal(pws[0].s, pws[1].s)
    rows = np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 13)]))
    ref = O.merge_lowrank_int8(canon, m1, m2, 2.0, 1.0, seed=2 ** 40 + 1, rows=rows)
    dc, ds, _ = Q.unpack(pws[0])
    torch.cuda.synchronize()
    assert np.array_equal(dc[torch.from_numpy(rows).cuda()].cpu().numpy(), ref["codes"])
    assert np.array_equal(ds[torch.from_numpy(rows).cuda()].cpu().view(torch.int16).numpy().view(np.uint16),
                          ref["scales"])


def test_merge_subnormal_range_products():
    """beta = 0 and adapter factors near 2^-72: the products and the merged weights lie in
    the float32 subnormal range, where a product rounded on its own would differ from the
    fused multiply-add the definition uses; the codes must still match byte for byte."""
    import bit_weight_only_offline_amd as Q
    N, K, G, r = 40, 512, 64, 16
    canon, _, _ = _case(N, K, G, r, 13)
    rng = np.random.default_rng(14)
    m1 = S.to_bf16_values((rng.standard_normal((N, r)) * 2.0 ** -72).astype(np.float32))
    m2 = S.to_bf16_values((rng.standard_normal((r, K)) * 2.0 ** -72).astype(np.float32))
    assert np.all(np.abs(m1 @ m2) < 2.0 ** -126)
    for seed in (None, 4):
        pw = _packed(Q, canon, N, K, G)
        Q.int8_addmm_(pw, torch.from_numpy(m1).cuda().to(torch.bfloat16),
                      torch.from_numpy(m2).cuda().to(torch.bfloat16), alpha=1.0, beta=0.0, rounding_seed=seed)
        _check_equal(Q, pw, O.merge_lowrank_int8(canon, m1, m2, 1.0, 0.0, seed=seed), N, K, G)
