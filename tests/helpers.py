"""Shared helpers of the GPU tests: oracle canonical arrays -> device tensors."""
from __future__ import annotations

import numpy as np

import oracle as O

FMT_ID = {"int4": 0, "mxfp4": 1, "int8": 2, "cb4": 3}


def to_device(fmt: str, canon: dict, device="cuda"):
    """(codes, scales, aux) torch tensors in the canonical layout of include/qlinear.h."""
    import torch
    codes = torch.from_numpy(np.ascontiguousarray(canon["codes"])).to(device)
    if fmt == "int4":
        scales = torch.from_numpy(np.ascontiguousarray(canon["scales"])).to(device)
        z = canon.get("zeros")
        aux = None if z is None else torch.from_numpy(np.ascontiguousarray(z)).to(device)
    elif fmt == "mxfp4":
        scales = torch.from_numpy(np.ascontiguousarray(canon["scales"])).to(device)
        aux = None
    elif fmt == "int8":
        scales = torch.from_numpy(np.ascontiguousarray(canon["scales"]).view(np.int16)).to(device).view(torch.bfloat16)
        aux = None
    else:
        scales = torch.from_numpy(np.ascontiguousarray(canon["scales"]).view(np.int16)).to(device).view(torch.bfloat16)
        aux = np.asarray(canon["centroids"], dtype=np.float32)
    return codes, scales, aux


def bf16_tensor(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(torch.bfloat16)


def quantize(fmt: str, w: np.ndarray, group: int, symmetric: bool = True) -> dict:
    if fmt == "cb4":
        return O.quantize("cb4", w, centroids=O.lloyd_max_gaussian()[0])
    return O.quantize(fmt, w, group, symmetric=symmetric)


def rel_err(y: np.ndarray, yref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(yref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(y.astype(np.float64) - yref))) / rms
