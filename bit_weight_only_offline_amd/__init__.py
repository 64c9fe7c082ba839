"""Python binding of libqlinear.so, the MI355X weight-only low-bit linear layer.

Argument marshalling only: every function checks dtypes and shapes, allocates the
output with PyTorch on the input's device and passes raw pointers, sizes and the
current HIP stream to the C ABI declared in include/qlinear.h.  All arithmetic runs
in the library's HIP kernels.  There is no fallback: if the library is missing or no
GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "QL_INT4", "QL_MXFP4", "QL_INT8", "QL_CB4", "FORMATS", "QLinearError", "lib", "version",
    "PackedWeight", "packed_bytes", "quantize", "pack", "unpack", "dequant_tile", "workspace_bytes", "linear",
    "Schedule", "default_schedule", "tile_shapes", "workspace", "PackedExperts", "pack_experts",
    "grouped_workspace_bytes", "grouped_linear", "int8_addmm_", "quantize_activations", "a8_tile_shapes",
    "a8_workspace_bytes", "linear_a8", "noalloc_scratch_bytes", "linear_noalloc",
]

QL_INT4, QL_MXFP4, QL_INT8, QL_CB4 = 0, 1, 2, 3
FORMATS = {"int4": QL_INT4, "mxfp4": QL_MXFP4, "int8": QL_INT8, "cb4": QL_CB4}
_ACT = {None: 0, "none": 0, "swiglu": 1}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlinear.so")
_lib = None


class QLinearError(RuntimeError):
    """A non-zero ql_status from the library."""


class Schedule(ctypes.Structure):
    """ql_schedule: tile = compiled tile shape (-1 automatic), splits = k-splits (0 automatic)."""
    _fields_ = [("tile", ctypes.c_int32), ("splits", ctypes.c_int32)]

    def __repr__(self) -> str:
        return f"Schedule(tile={self.tile}, splits={self.splits})"


def lib() -> ctypes.CDLL:
    """Load libqlinear.so from the package directory (built by build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise QLinearError(f"{_LIB_PATH} is missing: build it with python -m bit_weight_only_offline_amd.build")
        L = ctypes.CDLL(_LIB_PATH)
        i64, sz, vp, ci = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
        L.qlinear_version.restype = ci
        L.qlinear_error_string.restype = ctypes.c_char_p
        L.qlinear_error_string.argtypes = [ci]
        L.qlinear_packed_bytes.restype = ci
        L.qlinear_packed_bytes.argtypes = [ci, i64, i64, ci, ci, ctypes.POINTER(sz), ctypes.POINTER(sz),
                                           ctypes.POINTER(sz)]
        L.qlinear_grouped_workspace_bytes.restype = ci
        L.qlinear_grouped_workspace_bytes.argtypes = [ci, i64, i64, i64, i64, ci, ctypes.POINTER(sz)]
        L.qlinear_grouped_forward.restype = ci
        L.qlinear_grouped_forward.argtypes = [vp, i64, vp, i64, i64, i64, vp, vp, vp, ci, ci, ci, vp, vp, ci, vp, sz, vp]
        L.qlinear_quantize.restype = ci
        L.qlinear_int8_addmm.restype = ci
        L.qlinear_quantize_activations.restype = ci
        L.qlinear_quantize_activations.argtypes = [vp, i64, i64, vp, vp, vp]
        L.qlinear_a8_workspace_bytes.restype = ci
        L.qlinear_a8_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, ctypes.POINTER(sz)]
        L.qlinear_a8_num_tiles.restype = ci
        L.qlinear_a8_tile_shape.restype = ci
        L.qlinear_a8_tile_shape.argtypes = [ci, ctypes.POINTER(ci), ctypes.POINTER(ci)]
        L.qlinear_forward_a8.restype = ci
        L.qlinear_forward_a8.argtypes = [vp, i64, i64, i64, vp, vp, ci, ci, vp, vp, ci, vp, sz, ci, vp]
        L.qlinear_int8_addmm.argtypes = [i64, i64, ci, vp, vp, vp, vp, i64, ctypes.c_float, ctypes.c_float, ci,
                                         ctypes.c_uint64, vp]
        L.qlinear_quantize.argtypes = [ci, i64, i64, ci, vp, vp, vp, vp, vp, vp]
        L.qlinear_pack.restype = ci
        L.qlinear_pack.argtypes = [ci, i64, i64, ci, vp, vp, vp, vp, vp, vp, vp]
        L.qlinear_unpack.restype = ci
        L.qlinear_unpack.argtypes = [ci, i64, i64, ci, ci, vp, vp, vp, vp, vp, vp, vp]
        L.qlinear_dequant_tile.restype = ci
        L.qlinear_dequant_tile.argtypes = [ci, i64, i64, ci, ci, vp, vp, vp, i64, i64, i64, i64, ci, vp, vp]
        L.qlinear_workspace_bytes.restype = ci
        L.qlinear_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, ci, ctypes.POINTER(sz)]
        L.qlinear_forward.restype = ci
        L.qlinear_forward.argtypes = [vp, i64, i64, i64, vp, vp, vp, ci, ci, ci, vp, ci, vp, ci, vp, sz, vp]
        L.qlinear_num_tiles.restype = ci
        L.qlinear_tile_shape.restype = ci
        L.qlinear_tile_shape.argtypes = [ci, ctypes.POINTER(ci), ctypes.POINTER(ci), ctypes.POINTER(ci)]
        L.qlinear_default_schedule.restype = ci
        L.qlinear_default_schedule.argtypes = [ci, i64, i64, i64, ci, ci, ctypes.POINTER(Schedule)]
        L.qlinear_workspace_bytes_ex.restype = ci
        L.qlinear_workspace_bytes_ex.argtypes = [ci, i64, i64, i64, ci, ci, ctypes.POINTER(Schedule),
                                                 ctypes.POINTER(sz)]
        L.qlinear_noalloc_scratch_bytes.restype = sz
        L.qlinear_noalloc_scratch_bytes.argtypes = []
        L.qlinear_forward_noalloc.restype = ci
        L.qlinear_forward_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, vp, ci, ci, ci, vp, ci, vp, ci, vp]
        L.qlinear_forward_ex.restype = ci
        L.qlinear_forward_ex.argtypes = [vp, i64, i64, i64, vp, vp, vp, ci, ci, ci, vp, ci, vp, ci, vp, sz,
                                         ctypes.POINTER(Schedule), vp]
        _lib = L
    return _lib


def version() -> int:
    return int(lib().qlinear_version())


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().qlinear_error_string(status).decode()
        raise QLinearError(f"{what}: {msg} (status {status})")


def _fmt(f) -> int:
    return FORMATS[f] if isinstance(f, str) else int(f)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(device) -> torch.device:
    d = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if d.type != "cuda":
        raise QLinearError("the library runs on a HIP device only")
    return d


@dataclass
class PackedWeight:
    """A weight in the device layout (three uint8 device buffers) plus its shape."""
    fmt: int
    N: int
    K: int
    group: int
    has_zeros: int
    w: torch.Tensor
    s: torch.Tensor
    aux: torch.Tensor | None

    @property
    def device(self) -> torch.device:
        return self.w.device


def packed_bytes(fmt, N: int, K: int, group: int, has_zeros: bool = False):
    """(w_bytes, s_bytes, aux_bytes) of the device layout."""
    w, s, a = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().qlinear_packed_bytes(_fmt(fmt), N, K, group, int(has_zeros), ctypes.byref(w), ctypes.byref(s),
                                      ctypes.byref(a)), "qlinear_packed_bytes")
    return w.value, s.value, a.value


def quantize(fmt, w: torch.Tensor, group: int = 128, symmetric: bool = True, levels=None):
    """Round-to-nearest quantisation of dense float32 device weights [N, K] into the
    canonical arrays (codes, scales, aux) that pack() takes: aux is the uint8 zero-points
    (asymmetric INT4), the 16 codebook levels as a CPU tensor (CB4) or None."""
    f = _fmt(fmt)
    if w.requires_grad:
        raise QLinearError("inference-only operator: inputs must not require grad")
    if w.device.type != "cuda":
        raise QLinearError("the library runs on a HIP device only")
    if w.dtype != torch.float32 or w.dim() != 2:
        raise QLinearError("w must be a float32 [N, K] tensor")
    w = w.contiguous()
    N, K = w.shape
    dev = w.device
    G = {QL_MXFP4: 32, QL_CB4: 0}.get(f, group)
    if f == QL_INT8:
        codes = torch.empty((N, K), dtype=torch.int8, device=dev)
    else:
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    if f == QL_INT4:
        scales = torch.empty((N, K // G), dtype=torch.float16, device=dev)
    elif f == QL_INT8:
        scales = torch.empty((N, K // G), dtype=torch.bfloat16, device=dev)
    elif f == QL_MXFP4:
        scales = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
    else:
        scales = torch.empty((N,), dtype=torch.bfloat16, device=dev)
    zeros = torch.empty((N, K // G), dtype=torch.uint8, device=dev) if (f == QL_INT4 and not symmetric) else None
    lv_ptr = None
    lv = None
    if f == QL_CB4:
        if levels is None:
            raise QLinearError("a codebook quantiser needs its 16 levels")
        lv = torch.as_tensor(levels, dtype=torch.float32).cpu().contiguous()
        if lv.numel() != 16:
            raise QLinearError("a codebook has 16 levels")
        lv_ptr = lv.data_ptr()
    _check(lib().qlinear_quantize(f, N, K, G, _ptr(w), lv_ptr, _ptr(codes), _ptr(scales), _ptr(zeros), _stream(dev)),
           "qlinear_quantize")
    return codes, scales, (lv if f == QL_CB4 else zeros)


def pack(fmt, N: int, K: int, group: int, codes: torch.Tensor, scales: torch.Tensor, aux=None) -> PackedWeight:
    """Pack canonical device tensors (see include/qlinear.h) into the device layout.

    codes: uint8 [N, K/2] (4-bit formats) or int8 [N, K] (INT8); scales: float16 [N, K/G]
    (INT4), bfloat16 [N, K/G] (INT8), uint8 [N, K/32] (MXFP4), bfloat16 [N] norms (CB4);
    aux: uint8 zeros [N, K/G] (INT4 with zero-point, device) or 16 float32 centroids
    (CB4, host sequence or CPU tensor)."""
    f = _fmt(fmt)
    dev = codes.device
    has_zeros = 1 if (f == QL_INT4 and aux is not None) else 0
    wb, sb, ab = packed_bytes(f, N, K, group, bool(has_zeros))
    w = torch.empty(wb, dtype=torch.uint8, device=dev)
    s = torch.empty(sb, dtype=torch.uint8, device=dev)
    a = torch.empty(ab, dtype=torch.uint8, device=dev) if ab else None
    codes = codes.contiguous()
    scales = scales.contiguous()
    aux_ptr = None
    keep = None
    if f == QL_CB4:
        keep = torch.as_tensor(aux, dtype=torch.float32).cpu().contiguous()
        if keep.numel() != 16:
            raise QLinearError("a codebook has 16 centroids")
        aux_ptr = keep.data_ptr()
    elif aux is not None:
        aux = aux.contiguous()
        aux_ptr = aux.data_ptr()
    _check(lib().qlinear_pack(f, N, K, group, _ptr(codes), _ptr(scales), aux_ptr, _ptr(w), _ptr(s), _ptr(a),
                              _stream(dev)), "qlinear_pack")
    return PackedWeight(f, N, K, group, has_zeros, w, s, a)


def int8_addmm_(pw: PackedWeight, mat1: torch.Tensor, mat2: torch.Tensor, alpha: float = 1.0, beta: float = 1.0,
                rounding_seed: int | None = None) -> PackedWeight:
    """In place: pw <- beta * pw + alpha * (mat1 @ mat2), requantised to INT8 in the same
    device buffers.  mat1 bf16 [N, r] (the adapter's B), mat2 bf16 [r, K] (its A).
    rounding_seed: None for nearest rounding, else an unsigned 64-bit seed for the
    stochastic choice between the two neighbouring codes.  Returns pw."""
    if pw.fmt != QL_INT8:
        raise QLinearError("the low-rank merge updates INT8 weights")
    for t in (mat1, mat2):
        if t.requires_grad:
            raise QLinearError("inference-only operator: inputs must not require grad")
        if t.device != pw.device:
            raise QLinearError("mat1 and mat2 must be on the weight's device")
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise QLinearError("mat1 and mat2 must be bf16 matrices")
    r = mat1.shape[1]
    if tuple(mat1.shape) != (pw.N, r) or tuple(mat2.shape) != (r, pw.K):
        raise QLinearError(f"mat1 must be [N, r] and mat2 [r, K]; got {tuple(mat1.shape)} and {tuple(mat2.shape)}")
    if rounding_seed is not None and not 0 <= int(rounding_seed) < 2 ** 64:
        raise QLinearError("rounding_seed must be an unsigned 64-bit integer")
    m1, m2 = mat1.contiguous(), mat2.contiguous()
    _check(lib().qlinear_int8_addmm(pw.N, pw.K, pw.group, _ptr(pw.w), _ptr(pw.s), _ptr(m1) if r else None,
                                    _ptr(m2) if r else None, r,
                                    float(alpha), float(beta), 0 if rounding_seed is None else 1,
                                    0 if rounding_seed is None else int(rounding_seed), _stream(pw.device)),
           "qlinear_int8_addmm")
    return pw


def unpack(pw: PackedWeight):
    """Device layout -> canonical (codes, scales, aux) device tensors."""
    f, N, K, G = pw.fmt, pw.N, pw.K, pw.group
    dev = pw.device
    if f == QL_INT8:
        codes = torch.empty((N, K), dtype=torch.int8, device=dev)
    else:
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    if f == QL_INT4:
        scales = torch.empty((N, K // G), dtype=torch.float16, device=dev)
    elif f == QL_INT8:
        scales = torch.empty((N, K // G), dtype=torch.bfloat16, device=dev)
    elif f == QL_MXFP4:
        scales = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
    else:
        scales = torch.empty((N,), dtype=torch.bfloat16, device=dev)
    aux = None
    if f == QL_INT4 and pw.has_zeros:
        aux = torch.empty((N, K // G), dtype=torch.uint8, device=dev)
    elif f == QL_CB4:
        aux = torch.empty((16,), dtype=torch.float32, device=dev)
    _check(lib().qlinear_unpack(f, N, K, G, pw.has_zeros, _ptr(pw.w), _ptr(pw.s), _ptr(pw.aux), _ptr(codes),
                                _ptr(scales), _ptr(aux), _stream(dev)), "qlinear_unpack")
    return codes, scales, aux


def dequant_tile(pw: PackedWeight, n0: int = 0, k0: int = 0, tn: int | None = None, tk: int | None = None,
                 mode: int = 0) -> torch.Tensor:
    """float32 [tn, tk] dump of D(W) (mode 0) or of the bf16 matrix-core operand (mode 1)."""
    tn = pw.N - n0 if tn is None else tn
    tk = pw.K - k0 if tk is None else tk
    out = torch.empty((tn, tk), dtype=torch.float32, device=pw.device)
    _check(lib().qlinear_dequant_tile(pw.fmt, pw.N, pw.K, pw.group, pw.has_zeros, _ptr(pw.w), _ptr(pw.s),
                                      _ptr(pw.aux), n0, k0, tn, tk, mode, _ptr(out), _stream(pw.device)),
           "qlinear_dequant_tile")
    return out


def _sched(schedule):
    if schedule is None:
        return None
    if isinstance(schedule, Schedule):
        return ctypes.byref(schedule)
    tile, splits = schedule
    return ctypes.byref(Schedule(int(tile), int(splits)))


def workspace_bytes(fmt, M: int, N: int, K: int, group: int, act=None, schedule=None) -> int:
    b = ctypes.c_size_t()
    _check(lib().qlinear_workspace_bytes_ex(_fmt(fmt), M, N, K, group, _ACT[act], _sched(schedule),
                                            ctypes.byref(b)), "qlinear_workspace_bytes")
    return b.value


def default_schedule(fmt, M: int, N: int, K: int, group: int, act=None) -> Schedule:
    s = Schedule()
    _check(lib().qlinear_default_schedule(_fmt(fmt), M, N, K, group, _ACT[act], ctypes.byref(s)),
           "qlinear_default_schedule")
    return s


def tile_shapes():
    """[(rows, cols, kblock)] of the compiled tile shapes, by tile index."""
    out = []
    for t in range(lib().qlinear_num_tiles()):
        r, c, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(lib().qlinear_tile_shape(t, ctypes.byref(r), ctypes.byref(c), ctypes.byref(k)), "qlinear_tile_shape")
        out.append((r.value, c.value, k.value))
    return out


_WS = {}


def workspace(device, nbytes: int) -> torch.Tensor:
    """A shared workspace of at least nbytes on device, reused across calls on the
    device's current stream (the library does not depend on its contents on entry).

    There is one per (device, stream): calls on one stream run in order, so they may share
    it, while calls on two streams may overlap and must not.  It is allocated while that
    stream is current, so when it grows, the old buffer goes back to torch's allocator
    ordered after the work already queued on the stream."""
    d = torch.device(device)
    if d.index is None:
        d = torch.device(d.type, torch.cuda.current_device())
    key = (d.type, d.index, torch.cuda.current_stream(d).cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=d)
        _WS[key] = ws
    return ws


_shared_workspace = workspace


def linear(x: torch.Tensor, pw: PackedWeight, bias: torch.Tensor | None = None, act=None,
           out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, schedule=None) -> torch.Tensor:
    """Y = A . D(Wq)^T + b for bf16 x [..., K] (or [..., 2K] = [up | gate] with act="swiglu").

    workspace: a uint8 device buffer (any contents) that stays owned by the caller and
    may be reused (a shared one per device is used when omitted).  schedule: (tile,
    splits) or a Schedule to override the automatic choice.  Inference only: inputs that
    require grad are rejected."""
    if x.requires_grad or (bias is not None and bias.requires_grad):
        raise QLinearError("inference-only operator: inputs must not require grad")
    if x.device.type != "cuda" or pw.w.device.type != "cuda":
        raise QLinearError("the library runs on a HIP device only")
    if x.dtype != torch.bfloat16:
        raise QLinearError("x must be bfloat16")
    act_id = _ACT[act]
    width = 2 * pw.K if act_id == 1 else pw.K
    if x.shape[-1] != width:
        raise QLinearError(f"x has {x.shape[-1]} features, expected {width}")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, width)
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    M = x2.shape[0]
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != pw.N):
        raise QLinearError("bias must be bfloat16 [N]")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise QLinearError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((M, pw.N), dtype=out_dtype, device=x.device)
    elif out.dtype != out_dtype or out.numel() != M * pw.N or not out.is_contiguous() or out.device != x.device:
        raise QLinearError("out must be a contiguous [M, N] tensor of out_dtype on x's device")
    ws_need = workspace_bytes(pw.fmt, M, pw.N, pw.K, pw.group, act, schedule)
    if ws_need:
        if workspace is None:
            workspace = _shared_workspace(x.device, ws_need)
        elif workspace.numel() < ws_need or workspace.device != x.device:
            raise QLinearError(f"workspace needs {ws_need} bytes on {x.device}")
    _check(lib().qlinear_forward_ex(_ptr(x2), M, pw.N, pw.K, _ptr(pw.w), _ptr(pw.s), _ptr(pw.aux), pw.fmt,
                                    pw.group, pw.has_zeros, _ptr(bias), act_id, _ptr(out),
                                    1 if out_dtype == torch.float32 else 0,
                                    _ptr(workspace) if ws_need else None, ws_need if ws_need else 0,
                                    _sched(schedule), _stream(x.device)), "qlinear_forward")
    return out.reshape(*lead, pw.N)


def noalloc_scratch_bytes() -> int:
    """Bytes of the library's per-GPU scratch that linear_noalloc() uses as workspace."""
    return int(lib().qlinear_noalloc_scratch_bytes())


def linear_noalloc(x: torch.Tensor, pw: PackedWeight, bias: torch.Tensor | None = None, act=None,
                   out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """linear() through qlinear_forward_noalloc: the library's per-GPU scratch serves as
    workspace, so the call itself allocates nothing on the device (pass `out` to keep the
    wrapper from allocating the output).  Calls that overlap on one GPU share the scratch."""
    if x.requires_grad or (bias is not None and bias.requires_grad):
        raise QLinearError("inference-only operator: inputs must not require grad")
    if x.device.type != "cuda" or pw.w.device.type != "cuda":
        raise QLinearError("the library runs on a HIP device only")
    if x.dtype != torch.bfloat16:
        raise QLinearError("x must be bfloat16")
    act_id = _ACT[act]
    width = 2 * pw.K if act_id == 1 else pw.K
    if x.shape[-1] != width or not x.is_contiguous():
        raise QLinearError(f"x must be a contiguous [..., {width}] tensor")
    lead = x.shape[:-1]
    M = x.numel() // width
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != pw.N):
        raise QLinearError("bias must be bfloat16 [N]")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise QLinearError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((M, pw.N), dtype=out_dtype, device=x.device)
    elif out.dtype != out_dtype or out.numel() != M * pw.N or not out.is_contiguous() or out.device != x.device:
        raise QLinearError("out must be a contiguous [M, N] tensor of out_dtype on x's device")
    _check(lib().qlinear_forward_noalloc(_ptr(x), M, pw.N, pw.K, _ptr(pw.w), _ptr(pw.s), _ptr(pw.aux), pw.fmt,
                                         pw.group, pw.has_zeros, _ptr(bias), act_id, _ptr(out),
                                         1 if out_dtype == torch.float32 else 0, _stream(x.device)),
           "qlinear_forward_noalloc")
    return out.reshape(*lead, pw.N)


@dataclass
class PackedExperts:
    """E experts' packed weights back to back in one set of device buffers."""
    fmt: int
    E: int
    N: int
    K: int
    group: int
    has_zeros: int
    w: torch.Tensor
    s: torch.Tensor
    aux: torch.Tensor | None

    @property
    def device(self) -> torch.device:
        return self.w.device


def pack_experts(fmt, N: int, K: int, group: int, experts) -> PackedExperts:
    """Pack E experts, each given as canonical (codes, scales, aux) device tensors (aux as
    for pack()), into consecutive slices of one set of buffers."""
    f = _fmt(fmt)
    experts = list(experts)
    E = len(experts)
    if E == 0:
        raise QLinearError("no experts")
    dev = experts[0][0].device
    has_zeros = 1 if (f == QL_INT4 and experts[0][2] is not None) else 0
    wb, sb, ab = packed_bytes(f, N, K, group, bool(has_zeros))
    w = torch.empty(E * wb, dtype=torch.uint8, device=dev)
    s = torch.empty(E * sb, dtype=torch.uint8, device=dev)
    a = torch.empty(E * ab, dtype=torch.uint8, device=dev) if ab else None
    keep = []
    for e, (codes, scales, aux) in enumerate(experts):
        codes = codes.contiguous()
        scales = scales.contiguous()
        aux_ptr = None
        if f == QL_CB4:
            lv = torch.as_tensor(aux, dtype=torch.float32).cpu().contiguous()
            keep.append(lv)
            aux_ptr = lv.data_ptr()
        elif aux is not None:
            aux = aux.contiguous()
            keep.append(aux)
            aux_ptr = aux.data_ptr()
        _check(lib().qlinear_pack(f, N, K, group, _ptr(codes), _ptr(scales), aux_ptr, w.data_ptr() + e * wb,
                                  s.data_ptr() + e * sb, None if a is None else a.data_ptr() + e * ab, _stream(dev)),
               "qlinear_pack")
    return PackedExperts(f, E, N, K, group, has_zeros, w, s, a)


def grouped_workspace_bytes(fmt, T: int, E: int, N: int, K: int, group: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().qlinear_grouped_workspace_bytes(_fmt(fmt), T, E, N, K, group, ctypes.byref(n)),
           "qlinear_grouped_workspace_bytes")
    return n.value


def grouped_linear(x: torch.Tensor, pe: PackedExperts, tokens_per_expert: torch.Tensor, bias=None,
                   out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Mixture-of-experts linear: rows of x [T, K] grouped by expert in expert order,
    tokens_per_expert an int32 device tensor [E]; bias bf16 [E, N] or None.  Rows past
    the sum of the counts are left as they are in `out` (uninitialised when allocated)."""
    if x.requires_grad or (bias is not None and bias.requires_grad):
        raise QLinearError("inference-only operator: inputs must not require grad")
    if x.device.type != "cuda" or pe.w.device.type != "cuda" or tokens_per_expert.device.type != "cuda":
        raise QLinearError("the library runs on a HIP device only")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != pe.K:
        raise QLinearError("x must be bfloat16 [T, K]")
    if tokens_per_expert.dtype != torch.int32 or tokens_per_expert.numel() != pe.E:
        raise QLinearError("tokens_per_expert must be int32 [E]")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != pe.E * pe.N):
        raise QLinearError("bias must be bfloat16 [E, N]")
    x = x.contiguous()
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, pe.N), dtype=out_dtype, device=x.device)
    nbytes = grouped_workspace_bytes(pe.fmt, T, pe.E, pe.N, pe.K, pe.group)
    if workspace is None:
        workspace = _shared_workspace(x.device, nbytes)
    elif workspace.numel() < nbytes or workspace.device != x.device:
        raise QLinearError(f"workspace needs {nbytes} bytes on {x.device}")
    od = 1 if out_dtype == torch.float32 else 0
    _check(lib().qlinear_grouped_forward(_ptr(x), T, _ptr(tokens_per_expert.contiguous()), pe.E, pe.N, pe.K,
                                         _ptr(pe.w), _ptr(pe.s), _ptr(pe.aux), pe.fmt, pe.group, pe.has_zeros,
                                         _ptr(bias), _ptr(out), od, _ptr(workspace), workspace.numel(),
                                         _stream(x.device)), "qlinear_grouped_forward")
    return out



# ---- INT8-compute path (W4A8 / W8A8): dynamic per-row activation quantisation ----------

def quantize_activations(x: torch.Tensor):
    """Per-row symmetric INT8 quantisation of bf16 activations [M, K]:
    -> (codes int8 [M, K], scales float32 [M]), s = amax / 127, q = rint(x / s)."""
    if x.requires_grad:
        raise QLinearError("inference-only operator: inputs must not require grad")
    if x.device.type != "cuda" or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise QLinearError("x must be a bf16 [M, K] device tensor")
    x = x.contiguous()
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.int8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().qlinear_quantize_activations(_ptr(x), M, K, _ptr(codes), _ptr(scales), _stream(x.device)),
           "qlinear_quantize_activations")
    return codes, scales


def a8_tile_shapes():
    """[(rows, cols)] of the INT8-compute kernel's compiled schedules."""
    out = []
    for t in range(lib().qlinear_a8_num_tiles()):
        r, c = ctypes.c_int(), ctypes.c_int()
        _check(lib().qlinear_a8_tile_shape(t, ctypes.byref(r), ctypes.byref(c)), "qlinear_a8_tile_shape")
        out.append((r.value, c.value))
    return out


def a8_workspace_bytes(fmt, M: int, N: int, K: int, group: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().qlinear_a8_workspace_bytes(_fmt(fmt), M, N, K, group, ctypes.byref(n)), "qlinear_a8_workspace_bytes")
    return n.value


def linear_a8(x: torch.Tensor, pw: PackedWeight, bias: torch.Tensor | None = None, out_dtype=torch.bfloat16,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, tile: int | None = None):
    """Y = dequant(quantise_int8(x)) . D(W)^T + bias on the INT8 matrix cores, for symmetric
    INT4 or INT8 packed weights (group >= 64).  x bf16 [..., K]; tile None = automatic."""
    if x.requires_grad or (bias is not None and bias.requires_grad):
        raise QLinearError("inference-only operator: inputs must not require grad")
    if x.device.type != "cuda" or x.dtype != torch.bfloat16:
        raise QLinearError("x must be a bf16 device tensor")
    if x.shape[-1] != pw.K:
        raise QLinearError(f"x has {x.shape[-1]} inputs, the weight {pw.K}")
    if pw.has_zeros:
        raise QLinearError("the INT8-compute path takes symmetric weights")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, pw.K).contiguous()
    M = x2.shape[0]
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise QLinearError("out_dtype must be bf16 or float32")
    if out is None:
        out = torch.empty((M, pw.N), dtype=out_dtype, device=x.device)
    elif out.dtype != out_dtype or out.numel() != M * pw.N or not out.is_contiguous():
        raise QLinearError("out must be a contiguous [M, N] tensor of out_dtype")
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.numel() != pw.N:
            raise QLinearError("bias must be bf16 [N]")
        bias = bias.contiguous()
    need = a8_workspace_bytes(pw.fmt, M, pw.N, pw.K, pw.group)
    if workspace is None:
        workspace = _shared_workspace(x.device, need)
    od = 1 if out_dtype == torch.float32 else 0
    _check(lib().qlinear_forward_a8(_ptr(x2), M, pw.N, pw.K, _ptr(pw.w), _ptr(pw.s), pw.fmt, pw.group, _ptr(bias),
                                    _ptr(out), od, _ptr(workspace), workspace.numel(),
                                    -1 if tile is None else int(tile), _stream(x.device)), "qlinear_forward_a8")
    return out.reshape(*lead, pw.N)
