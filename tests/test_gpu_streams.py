"""Calls on two streams at once through the Python binding's shared workspace.

A schedule with split-K partial sums, and the SwiGLU input materialised before the decode
kernel, both use the caller's workspace.  The binding keeps one shared workspace per
(device, stream), so calls queued on two streams that overlap on the GPU must each give
what they give alone.
"""
import numpy as np
import pytest

import synthetic as S
from helpers import quantize, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _bf16(rng, shape):
    return torch.from_numpy(S.to_bf16_values(rng.standard_normal(shape).astype(np.float32))).cuda().to(torch.bfloat16)


@pytest.mark.parametrize("M,act,sched", [(64, None, (12, 4)), (16, "swiglu", None)], ids=["splitk", "swiglu"])
def test_two_streams_share_nothing(M, act, sched):
    import bit_weight_only_offline_amd as Q
    rng = np.random.default_rng(M)
    N, K, G = 1024, 2048, 128
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    pw = Q.pack("int4", N, K, G, *to_device("int4", quantize("int4", w, G, True)))
    width = 2 * K if act else K
    xs = [_bf16(rng, (M, width)) for _ in range(2)]
    refs = [Q.linear(x, pw, act=act, schedule=sched).clone() for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(5):
        print(f"two streams M={M} act={act} rep={rep}", flush=True)
        ys = []
        for s, x in zip(streams, xs):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                ys.append(Q.linear(x, pw, act=act, schedule=sched))
        torch.cuda.synchronize()
        for y, ref in zip(ys, refs):
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
