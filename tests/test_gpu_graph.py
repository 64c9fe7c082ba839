"""Entry points captured in a HIP graph and replayed.

Every entry point is asynchronous on the caller's stream and records no memset, so a
captured call must give, at every replay, exactly what the same call gives eagerly on the
inputs current at that replay.  Each case captures one call, then three times over: writes
new inputs in place, runs unrelated eager work through the library (another shape, the
shared workspace), replays the graph, and compares the replay's outputs with an eager
call on the same inputs, bit for bit.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import quantize, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


def _bf16(rng, shape, std=1.0):
    return torch.from_numpy(S.to_bf16_values((rng.standard_normal(shape) * std).astype(np.float32))).cuda().to(
        torch.bfloat16)


def _packed(fmt, G, sym, N, K, seed):
    import bit_weight_only_offline_amd as Q
    w = (np.random.default_rng(seed).standard_normal((N, K)) * 0.02).astype(np.float32)
    return Q.pack(fmt, N, K, G, *to_device(fmt, quantize(fmt, w, G, sym)))


def _other_work(Q, rng):
    """Unrelated eager library work between replays (its own shapes and the shared
    workspace), so a replay cannot lean on state the capture left behind."""
    pw = _packed("int4", 128, True, 96, 512, int(rng.integers(1 << 30)))
    x = _bf16(rng, (40, 512))
    Q.linear(x, pw, schedule=(12, 2))
    Q.linear(x[:3], pw)


def _graph(fn):
    """Capture fn() (after one eager warm-up on the capture stream) and return the graph
    and the tensors the captured call wrote."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def _same(a, b):
    assert a.shape == b.shape and a.dtype == b.dtype
    assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


# (format, group, symmetric, M, N, K, act, schedule): the decode kernel, the ring tiles with
# and without split-K (then the reduce kernel), the SwiGLU input formed by the decode
# kernel itself (one row) and materialised by the prologue
LINEAR = [
    ("int4", 128, False, 16, 512, 4096, None, None),
    ("int4", 64, True, 200, 320, 1024, None, None),
    ("mxfp4", 32, True, 64, 512, 2048, None, (12, 4)),
    ("int8", 256, True, 1, 256, 2048, "swiglu", None),
    ("int8", 256, True, 16, 256, 2048, "swiglu", None),
    ("int8", 256, True, 130, 256, 1024, "swiglu", None),
    ("cb4", 0, True, 300, 384, 768, None, None),
]


@pytest.mark.parametrize("case", LINEAR, ids=[f"{c[0]}_m{c[3]}{'_swiglu' if c[6] else ''}{'_splitk' if c[7] else ''}"
                                              for c in LINEAR])
def test_linear_replays_match_eager(case):
    import bit_weight_only_offline_amd as Q
    fmt, G, sym, M, N, K, act, sched = case
    print(f"graph linear {case}", flush=True)
    rng = np.random.default_rng(M + N + K)
    pw = _packed(fmt, G, sym, N, K, seed=N * K)
    width = 2 * K if act else K
    x = _bf16(rng, (M, width))
    bias = _bf16(rng, (N,), 0.01)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(Q.workspace_bytes(fmt, M, N, K, G, act, sched), 256), dtype=torch.uint8, device="cuda")
    g, _ = _graph(lambda: Q.linear(x, pw, bias=bias, act=act, out=out, workspace=ws, schedule=sched))
    for r in range(REPLAYS):
        x.copy_(_bf16(rng, (M, width)))
        _other_work(Q, rng)
        ref = Q.linear(x, pw, bias=bias, act=act, schedule=sched).clone()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _same(out, ref)


def test_grouped_replays_follow_device_counts():
    """The routing plan is built on the device from the counts at each replay, so changing
    the counts in place between replays reroutes the captured call."""
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(11)
    E, N, K, T = 4, 256, 512, 96
    dev = []
    for e in range(E):
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        dev.append(to_device("int4", quantize("int4", w, 128, False)))
    pe = Q.pack_experts("int4", N, K, 128, dev)
    x = _bf16(rng, (T, K))
    bias = _bf16(rng, (E, N), 0.01)
    cnt = torch.tensor([T, 0, 0, 0], dtype=torch.int32, device="cuda")
    out = torch.zeros((T, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(Q.grouped_workspace_bytes("int4", T, E, N, K, 128), dtype=torch.uint8, device="cuda")
    g, _ = _graph(lambda: Q.grouped_linear(x, pe, cnt, bias=bias, out=out, workspace=ws))
    for counts in ([10, 50, 0, 36], [1, 1, 1, 93], [40, 40, 16, 0]):
        cnt.copy_(torch.tensor(counts, dtype=torch.int32))
        x.copy_(_bf16(rng, (T, K)))
        _other_work(Q, rng)
        ref = Q.grouped_linear(x, pe, cnt, bias=bias).clone()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        _same(out, ref)


@pytest.mark.parametrize("fmt,G", [("int4", 128), ("int8", 256)])
def test_linear_a8_replays_match_eager(fmt, G):
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(G)
    M, N, K = 72, 320, 1024
    pw = _packed(fmt, G, True, N, K, seed=7)
    x = _bf16(rng, (M, K))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(Q.a8_workspace_bytes(fmt, M, N, K, G), dtype=torch.uint8, device="cuda")
    g, _ = _graph(lambda: Q.linear_a8(x, pw, out=out, workspace=ws))
    for r in range(REPLAYS):
        x.copy_(_bf16(rng, (M, K)))
        _other_work(Q, rng)
        ref = Q.linear_a8(x, pw).clone()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _same(out, ref)


@pytest.mark.parametrize("seed", [None, 1234])
def test_int8_addmm_replays_match_eager(seed):
    """A captured in-place merge applied by each replay equals the same number of eager
    merges (nearest, or stochastic with a fixed seed: the same codes every time)."""
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(3)
    N, K, r = 64, 1024, 16
    a = _packed("int8", 256, True, N, K, seed=5)
    b = _packed("int8", 256, True, N, K, seed=5)
    m1 = _bf16(rng, (N, r), 0.05)
    m2 = _bf16(rng, (r, K), 0.05)
    g, _ = _graph(lambda: Q.int8_addmm_(b, m1, m2, alpha=0.5, beta=0.9, rounding_seed=seed))
    Q.int8_addmm_(a, m1, m2, alpha=0.5, beta=0.9, rounding_seed=seed)     # the warm-up call on b
    for _ in range(REPLAYS):
        _other_work(Q, rng)
        Q.int8_addmm_(a, m1, m2, alpha=0.5, beta=0.9, rounding_seed=seed)
        g.replay()
        torch.cuda.synchronize()
        _same(b.w, a.w)
        _same(b.s, a.s)


@pytest.mark.parametrize("fmt,G,sym", [("int4", 128, False), ("mxfp4", 32, True), ("int8", 256, True),
                                       ("cb4", 0, True)])
def test_quantize_replays_match_eager(fmt, G, sym):
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(G + 1)
    N, K = 96, 512
    levels = O.lloyd_max_gaussian()[0] if fmt == "cb4" else None
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).cuda()
    g, outs = _graph(lambda: Q.quantize(fmt, w, G, sym, levels=levels))
    for _ in range(REPLAYS):
        w.copy_(torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)))
        _other_work(Q, rng)
        ref = Q.quantize(fmt, w, G, sym, levels=levels)
        g.replay()
        torch.cuda.synchronize()
        _same(outs[0], ref[0])
        _same(outs[1], ref[1])
        if fmt == "int4":
            _same(outs[2], ref[2])


_CAPTURE_FIRST = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import bit_weight_only_offline_amd as Q
import synthetic as S
from helpers import quantize, to_device

N, K, M = 200, 640, 300
w = (np.random.default_rng(5).standard_normal((N, K)) * 0.02).astype(np.float32)
pw = Q.pack("mxfp4", N, K, 32, *to_device("mxfp4", quantize("mxfp4", w, 32)))
x = torch.from_numpy(S.to_bf16_values(np.random.default_rng(6).standard_normal((M, K)).astype(np.float32))).cuda()
x = x.to(torch.bfloat16)
out = torch.empty((M, N), dtype=torch.float32, device="cuda")
ws = torch.zeros(max(Q.workspace_bytes("mxfp4", M, N, K, 32, None, (13, 2)), 256), dtype=torch.uint8, device="cuda")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):            # the first forward of this process, inside the capture
    Q.linear(x, pw, out_dtype=torch.float32, out=out, workspace=ws, schedule=(13, 2))
for _ in range(3):
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    ref = Q.linear(x, pw, out_dtype=torch.float32, schedule=(13, 2))
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "replay differs from the eager call"
print("capture-first ok", flush=True)
"""


def test_first_call_inside_a_capture():
    """A process whose very first forward (here a ring schedule with a split, so the
    kernel's dynamic-LDS limit is raised and a reduce kernel runs) happens inside a
    graph capture: the capture succeeds and every replay equals the eager call."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([root, os.path.join(root, "tests"), env.get("PYTHONPATH", "")])
    r = subprocess.run([sys.executable, "-c", _CAPTURE_FIRST, root], capture_output=True, text=True, timeout=240,
                       env=env)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "capture-first ok" in r.stdout
