"""The C-ABI library without a GPU: it loads, exports every entry point that
include/qlinear.h declares, sizes its buffers as documented and rejects invalid
arguments before queuing any work (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")

QL_OK, QL_E_ARG, QL_E_SHAPE, QL_E_ALIGN, QL_E_UNSUPPORTED, QL_E_WORKSPACE, QL_E_HIP = range(7)
INT4, MXFP4, INT8, CB4 = range(4)
FAKE = 1 << 20          # an aligned address that is never dereferenced


@pytest.fixture(scope="module")
def L():
    import bit_weight_only_offline_amd as Q
    return Q.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qlinear_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert L.qlinear_version() == 0x000100


def test_error_strings(L):
    for s in range(7):
        assert L.qlinear_error_string(s)
    assert L.qlinear_error_string(99) == b"unknown status"


def _sizes(L, f, N, K, G, z):
    w, s, a = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = L.qlinear_packed_bytes(f, N, K, G, z, ctypes.byref(w), ctypes.byref(s), ctypes.byref(a))
    return st, w.value, s.value, a.value


def test_packed_bytes_layout(L):
    # INT4 4096 x 4096, group 128 with zeros: 256 column tiles x 32 chunks x 1 KiB,
    # fp16 scales [256][32][16], 4-bit zeros [256][32][8 bytes]
    assert _sizes(L, INT4, 4096, 4096, 128, 1) == (QL_OK, 8388608, 262144, 65536)
    # MXFP4 28672 x 4096: one 32-bit word of four E8M0 codes per column and chunk
    assert _sizes(L, MXFP4, 28672, 4096, 32, 0) == (QL_OK, 1792 * 32 * 1024, 1792 * 32 * 64, 0)
    # INT8 8192 x 28672 group 256: chunks of 64 inputs, bf16 scales
    assert _sizes(L, INT8, 8192, 28672, 256, 0) == (QL_OK, 512 * 448 * 1024, 512 * 112 * 32, 0)
    # CB4 3072 x 3072: float32 row scales + bf16 norms, 128-byte codebook record
    assert _sizes(L, CB4, 3072, 3072, 0, 0) == (QL_OK, 192 * 24 * 1024, 3072 * 6, 128)
    # ragged N and K are padded to whole tiles / chunks (and 256-byte multiples)
    st, w, s, a = _sizes(L, INT4, 50, 448, 32, 1)
    assert st == QL_OK and w == 4 * 4 * 1024 and s == 4 * 16 * 32 and a == 512


@pytest.mark.parametrize("args,code", [
    ((7, 64, 64, 32, 0), QL_E_ARG),           # unknown format
    ((INT4, 64, 48, 32, 0), QL_E_SHAPE),      # K not a multiple of 32
    ((INT4, 64, 256, 48, 0), QL_E_SHAPE),     # unsupported group
    ((INT4, 64, 320, 128, 0), QL_E_SHAPE),    # K not a multiple of the group
    ((MXFP4, 64, 256, 64, 0), QL_E_SHAPE),    # MXFP4 blocks are 32
    ((INT8, 64, 256, 256, 1), QL_E_ARG),      # zero-points only for INT4
    ((INT4, 0, 256, 128, 0), QL_E_SHAPE),     # empty weight
    ((INT4, -5, 256, 128, 0), QL_E_SHAPE),
])
def test_packed_bytes_rejects(L, args, code):
    assert _sizes(L, *args)[0] == code


def _fwd(L, x=FAKE, M=4, N=64, K=256, w=FAKE, s=FAKE, aux=None, f=INT4, G=128, z=0, bias=None, act=0,
         out=FAKE, od=0, ws=None, wsb=0):
    return L.qlinear_forward(x, M, N, K, w, s, aux, f, G, z, bias, act, out, od, ws, wsb, None)


def test_forward_validation_before_launch(L):
    assert _fwd(L, M=0) == QL_OK                         # no-op
    assert _fwd(L, x=None) == QL_E_ARG
    assert _fwd(L, out=None) == QL_E_ARG
    assert _fwd(L, x=FAKE + 8) == QL_E_ALIGN             # x must be 16-byte aligned
    assert _fwd(L, out=FAKE + 1) == QL_E_ALIGN
    assert _fwd(L, act=5) == QL_E_ARG
    assert _fwd(L, od=3) == QL_E_ARG
    assert _fwd(L, M=-1) == QL_E_SHAPE
    assert _fwd(L, f=CB4, G=0, aux=None) == QL_E_ARG     # codebook record required
    assert _fwd(L, z=1, aux=None) == QL_E_ARG            # zero-points required
    # the 4096 x 4096 shape at M = 64 splits the input dimension over workgroups
    need = ctypes.c_size_t()
    assert L.qlinear_workspace_bytes(INT4, 64, 4096, 4096, 128, 0, ctypes.byref(need)) == QL_OK
    assert need.value > 0 and need.value % 256 == 0
    assert _fwd(L, M=64, N=4096, K=4096, ws=None, wsb=0) == QL_E_WORKSPACE
    assert _fwd(L, M=64, N=4096, K=4096, ws=FAKE, wsb=need.value - 1) == QL_E_WORKSPACE
    assert _fwd(L, M=64, N=4096, K=4096, ws=FAKE + 16, wsb=need.value + 64) == QL_E_ALIGN
    # decode shapes need no workspace, except the SwiGLU input materialised at decode
    assert L.qlinear_workspace_bytes(INT4, 16, 4096, 4096, 128, 0, ctypes.byref(need)) == QL_OK and need.value == 0
    assert L.qlinear_workspace_bytes(INT4, 16, 4096, 4096, 128, 1, ctypes.byref(need)) == QL_OK
    assert need.value == 16 * 4096 * 2
    assert _fwd(L, M=16, N=4096, K=4096, act=1, ws=None, wsb=0) == QL_E_WORKSPACE


def test_workspace_bytes_is_a_pure_function(L):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    for M in (1, 4, 8, 16, 64, 128, 2048):
        assert L.qlinear_workspace_bytes(INT8, M, 8192, 28672, 256, 1, ctypes.byref(a)) == QL_OK
        assert L.qlinear_workspace_bytes(INT8, M, 8192, 28672, 256, 1, ctypes.byref(b)) == QL_OK
        assert a.value == b.value
    assert L.qlinear_workspace_bytes(INT8, 0, 8192, 28672, 256, 0, ctypes.byref(a)) == QL_OK and a.value == 0


def test_pack_validation_before_launch(L):
    half = np.linspace(0.1, 2.0, 8).astype(np.float32)
    cent = np.concatenate([-half[::-1], half]).astype(np.float32)    # symmetric
    asym = cent.copy()
    asym[3] += 0.01
    assert L.qlinear_pack(CB4, 64, 256, 0, FAKE, FAKE, asym.ctypes.data, FAKE, FAKE, FAKE, None) == QL_E_UNSUPPORTED
    bad = cent.copy()
    bad[0] = np.inf
    assert L.qlinear_pack(CB4, 64, 256, 0, FAKE, FAKE, bad.ctypes.data, FAKE, FAKE, FAKE, None) == QL_E_UNSUPPORTED
    assert L.qlinear_pack(CB4, 64, 256, 0, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == QL_E_ARG
    assert L.qlinear_pack(INT8, 64, 256, 256, FAKE + 4, FAKE, None, FAKE, FAKE, None, None) == QL_E_ALIGN
    assert L.qlinear_pack(INT4, 64, 256, 128, FAKE, FAKE, None, FAKE + 8, FAKE, None, None) == QL_E_ALIGN
    assert L.qlinear_pack(MXFP4, 64, 256, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == QL_E_ARG
    assert L.qlinear_pack(INT4, 64, 256, 128, None, FAKE, None, FAKE, FAKE, None, None) == QL_E_ARG


def test_quantize_validation_before_launch(L):
    lv = np.linspace(-2.0, 2.0, 16).astype(np.float32)
    bad = lv.copy()
    bad[5] = np.nan
    F = QL_E_SHAPE
    assert L.qlinear_quantize(INT4, 64, 256, 100, FAKE, None, FAKE, FAKE, None, None) == F       # group
    assert L.qlinear_quantize(MXFP4, 64, 256, 64, FAKE, None, FAKE, FAKE, None, None) == F      # MX is 32
    assert L.qlinear_quantize(INT8, 64, 250, 256, FAKE, None, FAKE, FAKE, None, None) == F      # K % 32
    assert L.qlinear_quantize(CB4, 64, 256, 0, FAKE, None, FAKE, FAKE, None, None) == QL_E_ARG  # no levels
    assert L.qlinear_quantize(CB4, 64, 256, 0, FAKE, bad.ctypes.data, FAKE, FAKE, None, None) == QL_E_UNSUPPORTED
    assert L.qlinear_quantize(INT8, 64, 256, 256, FAKE, lv.ctypes.data, FAKE, FAKE, None, None) == QL_E_ARG
    assert L.qlinear_quantize(MXFP4, 64, 256, 32, FAKE, None, FAKE, FAKE, FAKE, None) == QL_E_ARG   # zeros
    assert L.qlinear_quantize(INT4, 64, 256, 128, None, None, FAKE, FAKE, None, None) == QL_E_ARG
    assert L.qlinear_quantize(INT4, 64, 256, 128, FAKE + 4, None, FAKE, FAKE, None, None) == QL_E_ALIGN
    assert L.qlinear_quantize(INT8, 64, 256, 256, FAKE, None, FAKE + 1, FAKE, None, None) == QL_E_ALIGN


def test_grouped_validation_before_launch(L):
    need = ctypes.c_size_t()
    assert L.qlinear_grouped_workspace_bytes(MXFP4, 256, 8, 4096, 14336, 32, ctypes.byref(need)) == QL_OK
    assert need.value > 0 and need.value % 256 == 0
    assert L.qlinear_grouped_workspace_bytes(MXFP4, 0, 8, 4096, 14336, 32, ctypes.byref(need)) == QL_OK
    assert need.value == 0

    def g(T=256, cnt=FAKE, E=8, N=4096, K=4096, w=FAKE, s=FAKE, aux=None, f=INT4, G=128, z=0, bias=None,
          out=FAKE, od=0, ws=FAKE, wsb=1 << 30):
        return L.qlinear_grouped_forward(FAKE, T, cnt, E, N, K, w, s, aux, f, G, z, bias, out, od, ws, wsb, None)

    assert g(T=0) == QL_OK and g(E=0) == QL_OK            # no-ops
    assert g(cnt=None) == QL_E_ARG
    assert g(cnt=FAKE + 2) == QL_E_ALIGN
    assert g(G=100) == QL_E_SHAPE
    assert g(T=-1) == QL_E_SHAPE
    assert g(od=2) == QL_E_ARG
    assert g(f=CB4, G=0) == QL_E_ARG                      # codebook record required
    assert g(ws=None, wsb=0) == QL_E_WORKSPACE
    assert g(ws=FAKE + 16) == QL_E_ALIGN


def test_dequant_tile_validation(L):
    assert L.qlinear_dequant_tile(INT4, 64, 256, 128, 0, FAKE, FAKE, None, 60, 0, 8, 8, 0, FAKE, None) == QL_E_SHAPE
    assert L.qlinear_dequant_tile(INT4, 64, 256, 128, 0, FAKE, FAKE, None, 0, 0, 8, 8, 2, FAKE, None) == QL_E_ARG
    assert L.qlinear_dequant_tile(INT4, 64, 256, 128, 0, FAKE, FAKE, None, 0, 0, 0, 8, 0, FAKE, None) == QL_OK


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import bit_weight_only_offline_amd as Q
    u8 = torch.zeros(256, dtype=torch.uint8)
    pw = Q.PackedWeight(Q.QL_INT4, 64, 256, 128, 0, u8, u8, None)
    with pytest.raises(Q.QLinearError, match="HIP device"):
        Q.linear(torch.zeros((1, 256), dtype=torch.bfloat16), pw)
    with pytest.raises(Q.QLinearError, match="grad"):
        Q.linear(torch.zeros((1, 256), dtype=torch.bfloat16, requires_grad=True), pw)


def test_schedule_entry_points(L):
    n = L.qlinear_num_tiles()
    assert n >= 4
    r, c, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    for t in range(n):
        assert L.qlinear_tile_shape(t, ctypes.byref(r), ctypes.byref(c), ctypes.byref(k)) == QL_OK
        assert r.value % 16 == 0 and c.value % 16 == 0 and k.value % 128 == 0
    assert L.qlinear_tile_shape(n, ctypes.byref(r), ctypes.byref(c), ctypes.byref(k)) == QL_E_ARG

    import bit_weight_only_offline_amd as Q
    Sched = Q.Schedule
    s = Sched()
    assert L.qlinear_default_schedule(INT4, 16, 4096, 4096, 128, 0, ctypes.byref(s)) == QL_OK
    assert 0 <= s.tile < n and s.splits >= 1
    b = ctypes.c_size_t()
    bad = Sched(n, 1)
    assert L.qlinear_workspace_bytes_ex(INT4, 16, 4096, 4096, 128, 0, ctypes.byref(bad), ctypes.byref(b)) == QL_E_ARG
    bad = Sched(0, -2)
    assert L.qlinear_workspace_bytes_ex(INT4, 16, 4096, 4096, 128, 0, ctypes.byref(bad), ctypes.byref(b)) == QL_E_ARG
    tile = [t for t in range(n) if L.qlinear_tile_shape(t, ctypes.byref(r), ctypes.byref(c), ctypes.byref(k)) == 0
            and k.value > 0][0]                          # first tile (not decode) schedule
    one = Sched(tile, 1)
    assert L.qlinear_workspace_bytes_ex(INT4, 16, 4096, 4096, 128, 0, ctypes.byref(one), ctypes.byref(b)) == QL_OK
    assert b.value == 0                                  # no split, no workspace
    four = Sched(tile, 4)
    assert L.qlinear_workspace_bytes_ex(INT4, 16, 4096, 4096, 128, 0, ctypes.byref(four), ctypes.byref(b)) == QL_OK
    assert b.value == 4 * 16 * 4096 * 4                  # 4 splits of float32 partial sums
    # groups of 256 span two 128-input chunks: splits are rounded to whole groups
    s7 = Sched(tile, 7)
    assert L.qlinear_workspace_bytes_ex(INT4, 1, 64, 1024, 256, 0, ctypes.byref(s7), ctypes.byref(b)) == QL_OK
    assert b.value == 4 * 1 * 64 * 4
    # a decode schedule serves M <= 16 and does not split over workgroups
    dec = Sched(0, 0)
    assert L.qlinear_workspace_bytes_ex(INT4, 17, 4096, 4096, 128, 0, ctypes.byref(dec), ctypes.byref(b)) == 4
    dec2 = Sched(0, 2)
    assert L.qlinear_workspace_bytes_ex(INT4, 8, 4096, 4096, 128, 0, ctypes.byref(dec2), ctypes.byref(b)) == 4


def test_decode_schedule_choice(L):
    """Decode schedules (M <= 16): the column tiles per workgroup follow the busiest
    compute unit's load (256 CUs); where the rows fit one activation load and there are
    four column tiles or more per CU, one tile per workgroup; and a single-tile workgroup
    over a long input dimension (eight wavefronts of 12 chunks or more) at up to 4 rows
    takes the four-deep ring instead of the two-deep one (same tile shape, another
    schedule)."""
    import bit_weight_only_offline_amd as Q
    r, c, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()

    def pick(fmt, M, N, K, G, act=0):
        s = Q.Schedule()
        assert L.qlinear_default_schedule(fmt, M, N, K, G, act, ctypes.byref(s)) == QL_OK
        assert L.qlinear_tile_shape(s.tile, ctypes.byref(r), ctypes.byref(c), ctypes.byref(k)) == QL_OK
        assert k.value == 0 and s.splits == 1            # the decode kernel: no split, no staging
        return s.tile, (r.value, c.value)

    # 4096 x 4096 INT4: one column tile per workgroup, four chunks per wavefront -> two-deep at every M
    t4 = {M: pick(INT4, M, 4096, 4096, 128) for M in (1, 4, 8, 16)}
    assert len({t for t, _ in t4.values()}) == 1 and t4[1][1] == (16, 16)
    # 4096 x 14336 MXFP4: 14 chunks per wavefront -> the four-deep schedule at M <= 4 only
    d1, d4, d16 = (pick(MXFP4, M, 4096, 14336, 32) for M in (1, 4, 16))
    assert d1 == d4 and d1[1] == d16[1] == (16, 16) and d1[0] != d16[0]
    assert d16[0] == t4[16][0]
    # 28672 x 4096 MXFP4 gate/up: 1792 column tiles -> seven per workgroup (256 workgroups),
    # but one per workgroup where the rows fit one activation load (four workgroups per CU)
    assert pick(MXFP4, 16, 28672, 4096, 32)[1] == (16, 112)
    assert pick(MXFP4, 1, 28672, 4096, 32)[1] == pick(MXFP4, 4, 28672, 4096, 32)[1] == (16, 16)
    assert pick(MXFP4, 5, 28672, 4096, 32)[1] == (16, 112)
    # 8192 x 28672 INT8 with the SwiGLU input: 512 column tiles -> two per workgroup
    assert pick(INT8, 1, 8192, 28672, 256, 1)[1] == (16, 32)


def test_launch_grid_limits(L):
    """Schedules whose launch grid exceeds the device's limits (65535 along the second
    and third grid dimensions, 2^31 - 1 along the first) are refused before any launch."""
    import bit_weight_only_offline_amd as Q
    Sched = Q.Schedule
    b = ctypes.c_size_t()
    r, c, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    n = L.qlinear_num_tiles()
    kinds = []
    for t in range(n):
        L.qlinear_tile_shape(t, ctypes.byref(r), ctypes.byref(c), ctypes.byref(k))
        kinds.append((t, r.value, c.value, k.value))
    ring = [t for t, rows, cols, kb in kinds if kb == 128][0]   # a ring tile (one chunk per stage)
    # splits along the grid's second dimension: 65535 are accepted, 65536 are not
    K = 65536 * 128
    ok = Sched(ring, 65535)
    assert L.qlinear_workspace_bytes_ex(CB4, 1, 16, K, 0, 0, ctypes.byref(ok), ctypes.byref(b)) == QL_OK
    over = Sched(ring, 65536)
    assert L.qlinear_workspace_bytes_ex(CB4, 1, 16, K, 0, 0, ctypes.byref(over), ctypes.byref(b)) == QL_E_UNSUPPORTED
    assert L.qlinear_forward_ex(FAKE, 1, 16, K, FAKE, FAKE, FAKE, CB4, 0, 0, None, 0, FAKE, 0, FAKE, 1 << 40,
                                ctypes.byref(over), None) == QL_E_UNSUPPORTED
    # grouped: ceil(T/16) + E decode slots past 65535 are served by the 32-row ring tile,
    # whose slot map (ceil(T/32) + E pairs of int32) sizes the workspace
    T = E = 70000
    assert L.qlinear_grouped_workspace_bytes(INT4, T, E, 16, 128, 128, ctypes.byref(b)) == QL_OK
    r256 = lambda v: (v + 255) // 256 * 256
    assert b.value == r256((E + 1) * 4) + r256(((T + 31) // 32 + E) * 8)
    T = E = 20000                                        # decode slots fit: 16-row slots
    assert L.qlinear_grouped_workspace_bytes(INT4, T, E, 16, 128, 128, ctypes.byref(b)) == QL_OK
    assert b.value == r256((E + 1) * 4) + r256(((T + 15) // 16 + E) * 8)
    # a ring grid of more than 2^31 - 1 workgroups
    assert L.qlinear_grouped_workspace_bytes(MXFP4, (1 << 31) - 1, 1, 1 << 20, 128, 32,
                                             ctypes.byref(b)) == QL_E_SHAPE


def test_int8_addmm_validation_before_launch(L):
    def a(N=64, K=256, G=256, w=FAKE, s=FAKE, m1=FAKE, m2=FAKE, r=8, alpha=1.0, beta=1.0, st=0, seed=0):
        return L.qlinear_int8_addmm(N, K, G, w, s, m1, m2, r, ctypes.c_float(alpha), ctypes.c_float(beta), st,
                                    ctypes.c_uint64(seed), None)

    assert a(G=100) == QL_E_SHAPE and a(K=250) == QL_E_SHAPE and a(K=128) == QL_E_SHAPE   # K % group
    assert a(N=0) == QL_E_SHAPE
    assert a(w=None) == QL_E_ARG and a(s=None) == QL_E_ARG
    assert a(m1=None) == QL_E_ARG and a(m2=None) == QL_E_ARG
    assert a(r=-1) == QL_E_ARG and a(r=257) == QL_E_ARG
    assert a(st=2) == QL_E_ARG
    assert a(alpha=float("nan")) == QL_E_ARG and a(beta=float("inf")) == QL_E_ARG
    assert a(w=FAKE + 8) == QL_E_ALIGN and a(s=FAKE + 4) == QL_E_ALIGN and a(m1=FAKE + 1) == QL_E_ALIGN


def test_a8_validation_before_launch(L):
    need = ctypes.c_size_t()
    assert L.qlinear_a8_workspace_bytes(INT4, 2048, 3072, 3072, 128, ctypes.byref(need)) == QL_OK
    assert need.value == 2048 * 3072 + 2048 * 4
    assert L.qlinear_a8_workspace_bytes(MXFP4, 16, 256, 256, 32, ctypes.byref(need)) == QL_E_UNSUPPORTED
    assert L.qlinear_a8_workspace_bytes(INT4, 16, 256, 256, 32, ctypes.byref(need)) == QL_E_UNSUPPORTED
    assert L.qlinear_a8_num_tiles() >= 1
    r, c = ctypes.c_int(), ctypes.c_int()
    assert L.qlinear_a8_tile_shape(L.qlinear_a8_num_tiles(), ctypes.byref(r), ctypes.byref(c)) == QL_E_ARG

    def f(M=64, N=256, K=256, fmt=INT4, G=128, x=FAKE, ws=FAKE, wsb=1 << 20, tile=-1, out=FAKE, od=0):
        return L.qlinear_forward_a8(x, M, N, K, FAKE, FAKE, fmt, G, None, out, od, ws, wsb, tile, None)

    assert f(M=0) == QL_OK
    assert f(fmt=CB4, G=0) == QL_E_UNSUPPORTED and f(G=32) == QL_E_UNSUPPORTED
    assert f(tile=99) == QL_E_ARG and f(tile=-2) == QL_E_ARG and f(od=5) == QL_E_ARG
    assert f(x=None) == QL_E_ARG and f(out=None) == QL_E_ARG
    assert f(ws=None) == QL_E_WORKSPACE and f(wsb=100) == QL_E_WORKSPACE
    assert f(x=FAKE + 8) == QL_E_ALIGN and f(ws=FAKE + 16) == QL_E_ALIGN
    assert L.qlinear_quantize_activations(FAKE, 4, 100, FAKE, FAKE, None) == QL_E_SHAPE
    assert L.qlinear_quantize_activations(FAKE + 2, 4, 128, FAKE, FAKE, None) == QL_E_ALIGN
    assert L.qlinear_quantize_activations(FAKE, 0, 128, None, None, None) == QL_OK
