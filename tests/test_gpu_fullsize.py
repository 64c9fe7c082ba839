"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The weights are the seeded synthetic weights of each workload at their real shape,
quantised by the oracle and packed on the device; the forward runs with the library's
default schedule (the one the benchmark uses).  The oracle computes a sample of the
outputs one by one (rows x columns including the first and last of each), which is
checked against the float32 output of the kernel (G2 on the sample, with the rms of
the sampled reference).  Properties that hold at any size are checked on the whole
output: the bf16 output is the RNE rounding of the float32 output (G3), two runs are
bit-identical, and no output is NaN or infinite.  The literal bf16 gate (G4) is printed
for each case next to the same figure for the correctly rounded bf16 of the exact
answer, which no bf16 output can beat.
"""
import zlib

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import quantize, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-2

WORKLOADS = [
    ("int4_asym_decode", (1, 4, 8, 16)),
    ("mxfp4_up", (1, 16, 64, 128, 512)),   # M = 128-512: the schedules of HBM-streamed weights
    ("mxfp4_down", (1, 16, 32, 64, 256)),
    ("int8_swiglu", (1, 16, 32, 128)),
    ("cb4_prefill", (256, 1024, 2048)),
]

_CACHE = {}


def _prepared(name):
    """Packed device weight + canonical arrays + inputs of one workload (built once)."""
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()                     # one full-size workload resident at a time
    import bit_weight_only_offline_amd as Q
    wl = S.WORKLOADS[name]
    fmt, N, K, G = wl["fmt"], wl["N"], wl["K"], wl["group"]
    canon = quantize(fmt, S.weights(wl), G, wl.get("symmetric", True))
    codes, scales, aux = to_device(fmt, canon)
    pw = Q.pack(fmt, N, K, G if fmt != "cb4" else 0, codes, scales, aux)
    del codes, scales
    x = S.activations(wl)
    b = S.bias(wl)
    _CACHE[name] = (wl, canon, pw, x, b)
    return _CACHE[name]


def _sample(M, N, rng):
    rows = np.arange(M) if M <= 16 else np.unique(np.concatenate([[0, 1, M // 2, M - 1], rng.integers(0, M, 12)]))
    cols = np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.integers(0, N, 60)]))
    return rows, cols


@pytest.mark.parametrize("name,M", [(n, m) for n, ms in WORKLOADS for m in ms],
                         ids=[f"{n}-M{m}" for n, ms in WORKLOADS for m in ms])
def test_full_size_sampled_parity(name, M):
    import bit_weight_only_offline_amd as Q
    wl, canon, pw, x_all, b = _prepared(name)
    if M > x_all.shape[0]:                 # beyond the workload's sweep: its leading rows extended
        x_all = S.activations(wl, M)
    fmt, N, K = wl["fmt"], wl["N"], wl["K"]
    swiglu = bool(wl.get("swiglu"))
    act = "swiglu" if swiglu else None
    print(f"full-size {name} M={M} N={N} K={K} schedule={Q.default_schedule(fmt, M, N, K, wl['group'], act)}",
          flush=True)
    x = torch.from_numpy(np.ascontiguousarray(x_all[:M])).cuda().to(torch.bfloat16)
    bias = None if b is None else torch.from_numpy(b).cuda().to(torch.bfloat16)

    y32 = Q.linear(x, pw, bias=bias, act=act, out_dtype=torch.float32)
    y16 = Q.linear(x, pw, bias=bias, act=act)
    y16b = Q.linear(x, pw, bias=bias, act=act)
    torch.cuda.synchronize()

    assert torch.isfinite(y32).all()
    assert torch.equal(y16.view(torch.int16), y16b.view(torch.int16)), "run-to-run difference"
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), "G3"

    rng = np.random.default_rng(zlib.crc32(f"{name}/{M}".encode()))
    rows, cols = _sample(M, N, rng)
    rr, cc = np.meshgrid(rows, cols, indexing="ij")
    ref = O.output_rows(fmt, x_all[:M], canon, K, rr.ravel(), cc.ravel(), bias=b, swiglu=swiglu)
    got = y32.cpu().numpy()[rr.ravel(), cc.ravel()].astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) / rms
    # G4: the bf16 output itself, and the correctly rounded bf16 of the exact answer
    got16 = y16.float().cpu().numpy()[rr.ravel(), cc.ravel()].astype(np.float64)
    g4 = float(np.max(np.abs(got16 - ref))) / rms
    g4_exact = float(np.max(np.abs(O.bf16_from_f64(ref).astype(np.float64) - ref))) / rms
    print(f"  sampled {len(ref)} outputs: G2 max|dY|/rms = {err:.3e}; G4 bf16 output {g4:.3e}, "
          f"correctly rounded exact answer {g4_exact:.3e}", flush=True)
    assert err <= TOL


def _record_split(pw) -> int:
    """The codebook record's operand choice (bytes 104..107): 1 = two-term operand."""
    return int(pw.aux.cpu().numpy()[104:108].view(np.uint32)[0])


@pytest.mark.parametrize("M", [256, 2048])
def test_codebook_dominant_rows_full_size(M):
    """The 3072 x 3072 codebook workload with four rows scaled by 100: those rows'
    outputs dominate rms(Y), so the single bf16 rounding of each level would show up in
    the gate; the packer sees the spread of the row norms and the kernels take the
    two-term operand.  The whole output is checked against the oracle (G2, G3)."""
    import bit_weight_only_offline_amd as Q
    wl = S.WORKLOADS["cb4_prefill"]
    N, K = wl["N"], wl["K"]
    w = S.weights(wl)
    rows = np.array([5, 700, 1901, 3070])
    w[rows] *= np.float32(100.0)
    canon = quantize("cb4", w, 0)
    codes, scales, aux = to_device("cb4", canon)
    pw = Q.pack("cb4", N, K, 0, codes, scales, aux)
    assert _record_split(pw) == 1
    x_all = S.activations(wl, M)
    b = S.bias(wl)
    print(f"codebook dominant rows M={M} schedule={Q.default_schedule('cb4', M, N, K, 0)}", flush=True)
    x = torch.from_numpy(np.ascontiguousarray(x_all)).cuda().to(torch.bfloat16)
    bias = torch.from_numpy(b).cuda().to(torch.bfloat16)
    y32 = Q.linear(x, pw, bias=bias, out_dtype=torch.float32)
    y16 = Q.linear(x, pw, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), "G3"
    ref = O.forward("cb4", x_all, canon, K, b)
    err = float(np.max(np.abs(y32.cpu().numpy().astype(np.float64) - ref))) / float(np.sqrt(np.mean(ref ** 2)))
    print(f"  whole output: G2 max|dY|/rms = {err:.3e}", flush=True)
    assert err <= TOL


def test_codebook_workload_keeps_one_term_operand():
    """The workload's own weights (row norms within a few percent of each other) keep the
    single bf16 operand: one MFMA per fragment."""
    _, _, pw, _, _ = _prepared("cb4_prefill")
    assert _record_split(pw) == 0
