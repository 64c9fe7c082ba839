"""Seeded synthetic inputs for the weight-only low-bit linear workloads.

This module is the only code that both the CPU oracle's tests and the HIP
library's tests, smoke check and benchmark use.  It holds random-number
generation, the workload shapes and nothing of the method's arithmetic: no
quantisation, packing, dequantisation, activation or matrix product.  Values
that must be bf16 (activations, bias) are drawn in float32 and truncated to the
nearest bf16 by a bit operation of this module's own; weights are returned as
float32 "master" values for a quantiser to consume.

Workloads (transformer-MLP shapes; every matrix is [out_features, in_features]):

* ``int4_sym_tiny``   INT4 symmetric, group 128, fp16 scales, bias.  X [4,512], W [512,512].
* ``int4_asym_decode`` INT4 with zero-point, group 128, fp16 scales + 4-bit zeros, no bias.
  X [M,4096] for M in {1,4,8,16}, W [4096,4096].
* ``mxfp4_up`` / ``mxfp4_down``  MXFP4 (E2M1 + E8M0 per 32).  W [28672,4096] and
  [4096,14336]; M in {1,16,64}; 0.1 % of weight positions (exactly round(0.001 N K),
  drawn without replacement) are multiplied by 20.
* ``int8_swiglu``  INT8 group 256, bf16 scales, bias, fused SwiGLU input.  Raw input
  [M, 2*28672] = [up | gate], W [8192,28672], M in {1,16,128}, W ~ N(0, 0.015).
* ``cb4_prefill``  4-bit Lloyd-Max codebook with bf16 row norms, bias.  X [M,3072],
  W [3072,3072], M in {256, 2048}.

X, up and gate ~ N(0,1); W ~ N(0, 0.02) unless stated; bias ~ N(0, 0.01).
Each workload's seed is split with numpy's SeedSequence into independent child
streams for weights, outlier positions, activations and bias, so an M sweep
shares its weights and a smaller M takes the leading rows of the largest M.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "int4_sym_tiny": dict(fmt="int4", symmetric=True, N=512, K=512, group=128,
                          Ms=(4,), seed=1, w_std=0.02, bias_std=0.01, swiglu=False),
    "int4_asym_decode": dict(fmt="int4", symmetric=False, N=4096, K=4096, group=128,
                             Ms=(1, 4, 8, 16), seed=2, w_std=0.02, bias_std=None, swiglu=False),
    "mxfp4_up": dict(fmt="mxfp4", N=28672, K=4096, group=32, Ms=(1, 16, 64), seed=3,
                     w_std=0.02, bias_std=None, swiglu=False, outlier_frac=0.001,
                     outlier_mult=20.0, stream=0),
    "mxfp4_down": dict(fmt="mxfp4", N=4096, K=14336, group=32, Ms=(1, 16, 64), seed=3,
                       w_std=0.02, bias_std=None, swiglu=False, outlier_frac=0.001,
                       outlier_mult=20.0, stream=1),
    "int8_swiglu": dict(fmt="int8", N=8192, K=28672, group=256, Ms=(1, 16, 128), seed=4,
                        w_std=0.015, bias_std=0.01, swiglu=True),
    "cb4_prefill": dict(fmt="cb4", N=3072, K=3072, group=0, Ms=(256, 2048), seed=5,
                        w_std=0.02, bias_std=0.01, swiglu=False),
}


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float32 data, returned as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def _streams(seed: int, n: int = 8):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _workload_streams(wl: dict):
    # Workloads that share a seed (the two MXFP4 shapes) take disjoint child streams.
    base = 4 * int(wl.get("stream", 0))
    s = _streams(int(wl["seed"]), base + 4)
    return s[base:base + 4]   # weights, outlier positions, activations, bias


def weights(wl: dict, N: int | None = None, K: int | None = None) -> np.ndarray:
    """float32 master weights [N, K] ~ N(0, w_std), with the workload's outliers."""
    N = wl["N"] if N is None else N
    K = wl["K"] if K is None else K
    g_w, g_o, _, _ = _workload_streams(wl)
    w = (g_w.standard_normal((N, K), dtype=np.float32) * np.float32(wl["w_std"])).astype(np.float32)
    frac = wl.get("outlier_frac")
    if frac:
        n_out = int(round(frac * N * K))
        pos = g_o.choice(N * K, size=n_out, replace=False)
        flat = w.reshape(-1)
        flat[pos] = flat[pos] * np.float32(wl["outlier_mult"])
    return w


def activations(wl: dict, M: int | None = None, K: int | None = None) -> np.ndarray:
    """bf16-valued float32 activations [M, K], or the raw [M, 2K] = [up | gate] input
    for a SwiGLU workload.  Rows are the leading rows of the largest M of the sweep."""
    K = wl["K"] if K is None else K
    Mmax = max(wl["Ms"]) if M is None else max(max(wl["Ms"]), M)
    M = Mmax if M is None else M
    _, _, g_x, _ = _workload_streams(wl)
    width = 2 * K if wl.get("swiglu") else K
    x = g_x.standard_normal((Mmax, width), dtype=np.float32)
    return to_bf16_values(x[:M])


def bias(wl: dict, N: int | None = None) -> np.ndarray | None:
    """bf16-valued float32 bias [N] ~ N(0, bias_std), or None."""
    if wl.get("bias_std") is None:
        return None
    N = wl["N"] if N is None else N
    _, _, _, g_b = _workload_streams(wl)
    return to_bf16_values(g_b.standard_normal(N, dtype=np.float32) * np.float32(wl["bias_std"]))


def small(name: str, N: int, K: int, seed_offset: int = 0) -> dict:
    """A reduced-size copy of a workload (same distributions, other shape and seed)."""
    wl = dict(WORKLOADS[name])
    wl.update(N=N, K=K, seed=int(wl["seed"]) * 1000 + 17 + seed_offset)
    return wl


def random_codes(rng: np.random.Generator, fmt: str, N: int, K: int, group: int,
                 symmetric: bool = False, w_std: float = 0.02):
    """Canonical-layout quantised weights drawn directly at random (no quantiser):
    for throughput measurement, where only the byte volume and a realistic spread of
    codes and scales matter.  Returns (codes, scales, aux) in the canonical layout:

    * int4:  uint8 [N, K/2] nibbles (two's complement if symmetric, else 0..15),
             fp16 scales [N, K/G], uint8 zeros [N, K/G] in 0..15 (None if symmetric)
    * mxfp4: uint8 [N, K/2] E2M1 nibbles, uint8 E8M0 scale codes [N, K/32]
    * int8:  int8 [N, K], bf16 scales as uint16 bits [N, K/G]
    * cb4:   uint8 [N, K/2] indices, bf16 row norms as uint16 bits [N], fp32 centroids
             from the caller (aux is None here)
    """
    packed = rng.integers(0, 256, size=(N, (K + 1) // 2), dtype=np.uint8)
    if fmt == "int4":
        G = group
        sc = (np.float32(w_std * 3.0 / 7.0) * rng.uniform(0.75, 1.25, (N, K // G))).astype(np.float16)
        zeros = None if symmetric else rng.integers(5, 11, size=(N, K // G), dtype=np.uint8)
        return packed, sc, zeros
    if fmt == "mxfp4":
        e = rng.integers(117, 122, size=(N, K // 32), dtype=np.uint8)
        return packed, e, None
    if fmt == "int8":
        codes = rng.integers(-127, 128, size=(N, K), dtype=np.int16).astype(np.int8)
        sc = to_bf16_values((np.float32(w_std * 3.5 / 127.0) * rng.uniform(0.75, 1.25, (N, K // group))).astype(np.float32))
        return codes, sc.view(np.uint32).__rshift__(16).astype(np.uint16), None
    if fmt == "cb4":
        nrm = to_bf16_values(np.full(N, np.float32(w_std * np.sqrt(K)), dtype=np.float32)
                             * rng.uniform(0.9, 1.1, N).astype(np.float32))
        return packed, (nrm.view(np.uint32) >> 16).astype(np.uint16), None
    raise ValueError(fmt)
