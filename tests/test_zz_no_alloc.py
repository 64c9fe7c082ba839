"""The allocation-free forward (qlinear_forward_noalloc) against qlinear_forward, through
the C ABI: the same kernels on the library's per-GPU scratch instead of a caller's
workspace, so the outputs are bit-identical.  Two calls in a row, the second with a
smaller input, for schedules that use the workspace (split-K partial sums, the
materialised SwiGLU input) and one that does not; a shape whose workspace exceeds the
scratch is refused before any launch and leaves the output untouched."""
import ctypes

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import quantize, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _packed(fmt, G, N, K, seed):
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    canon = quantize(fmt, w, G, True)
    codes, scales, aux = to_device(fmt, canon)
    return Q.pack(fmt, N, K, G, codes, scales, aux)


def _x(M, width, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(S.to_bf16_values(rng.standard_normal((M, width)).astype(np.float32))).cuda().to(
        torch.bfloat16)


def _noalloc(L, x, M, pw, bias, act, out, f32):
    st = torch.cuda.current_stream().cuda_stream
    return L.qlinear_forward_noalloc(x.data_ptr(), M, pw.N, pw.K, pw.w.data_ptr(), pw.s.data_ptr(),
                                     None if pw.aux is None else pw.aux.data_ptr(), pw.fmt, pw.group, pw.has_zeros,
                                     None if bias is None else bias.data_ptr(), act, out.data_ptr(), 1 if f32 else 0,
                                     st)


def _forward(L, x, M, pw, bias, act, out, f32):
    import bit_weight_only_offline_amd as Q
    nbytes = Q.workspace_bytes(pw.fmt, M, pw.N, pw.K, pw.group, "swiglu" if act else None)
    ws = torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    return L.qlinear_forward(x.data_ptr(), M, pw.N, pw.K, pw.w.data_ptr(), pw.s.data_ptr(),
                             None if pw.aux is None else pw.aux.data_ptr(), pw.fmt, pw.group, pw.has_zeros,
                             None if bias is None else bias.data_ptr(), act, out.data_ptr(), 1 if f32 else 0,
                             ws.data_ptr() if nbytes else None, nbytes, st), nbytes


# (format, group, N, K, act, M first, M second, uses the workspace)
CASES = [
    ("int4", 128, 300, 1024, 0, 40, 24, True),      # ring tiles with split-K: partial sums
    ("int8", 256, 256, 2048, 1, 16, 9, True),        # SwiGLU prologue: h in the workspace
    ("cb4", 0, 384, 768, 0, 300, 70, True),          # larger tiles, split-K
    ("mxfp4", 32, 512, 2048, 0, 8, 1, False),        # decode kernel: no workspace
    ("int8", 256, 256, 2048, 1, 2, 1, False),        # SwiGLU formed by the decode kernel
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_act{c[4]}_m{c[5]}_{c[6]}" for c in CASES])
def test_noalloc_matches_forward(case):
    import bit_weight_only_offline_amd as Q
    L = Q.lib()
    fmt, G, N, K, act, M1, M2, uses_ws = case
    print(f"noalloc {case}", flush=True)
    pw = _packed(fmt, G, N, K, seed=N + K)
    width = 2 * K if act else K
    bias = _x(1, N, 5).reshape(N)
    for i, M in enumerate((M1, M2)):
        x = _x(M, width, 10 * i + M)
        for f32 in (True, False):
            dt = torch.float32 if f32 else torch.bfloat16
            ref = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
            got = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
            st, nbytes = _forward(L, x, M, pw, bias, act, ref, f32)
            assert st == 0
            assert (nbytes > 0) == uses_ws or i == 1
            assert _noalloc(L, x, M, pw, bias, act, got, f32) == 0
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), (case, M, f32)
    # and through the binding
    x = _x(M2, width, 99)
    y = Q.linear_noalloc(x, pw, bias, act="swiglu" if act else None, out_dtype=torch.float32)
    y_ref = Q.linear(x, pw, bias, act="swiglu" if act else None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)


def test_noalloc_refuses_workspace_beyond_scratch():
    """SwiGLU at M = 2048, K = 28672: the materialised h alone is 112 MiB, more than the
    64 MiB scratch; the call is refused before any launch and the output keeps its bytes."""
    import bit_weight_only_offline_amd as Q
    L = Q.lib()
    N, K, M = 16, 28672, 2048
    assert Q.workspace_bytes("int8", M, N, K, 256, "swiglu") > L.qlinear_noalloc_scratch_bytes()
    pw = _packed("int8", 256, N, K, seed=3)
    x = torch.zeros((M, 2 * K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    assert _noalloc(L, x, M, pw, None, 1, out, True) == 5          # QL_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
