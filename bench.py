"""Benchmark of the weight-only low-bit linear layer on one MI355X.

One step = one forward of the INT4 decode workload with zero-points (group 128, fp16
scales, 4-bit zeros): X bf16 [16, 4096] times a packed 4096 x 4096 weight, bf16 out.
The metric is effective HBM bandwidth: algorithmic bytes (packed weight + scales +
zero-points + X + Y) per step over the step time.  Steps run back to back inside a
HIP graph (the launch-bound inner loop), each on the next copy of the packed weight
from a pool larger than four times the 256 MB Infinity Cache, timed with HIP events on
the stream the kernels run on.  Before every timed replay a 1 GiB buffer is read, so
the timed forwards find none of their weights in the caches, whatever the step count.

Also reported, on the same line (each leg timed the same way, with at least one forward
per pool copy in the graph, the clocks settled by 0.25 s of untimed replays, the median
of three timed replays):
  decode   every decode-sized workload: INT4 4096 x 4096 at M = 1, 4, 8, 16; MXFP4
           28672 x 4096 (gate/up) and 4096 x 14336 (down) at M = 1, 16; INT8 group
           256 with the fused SwiGLU input, 8192 x 28672, at M = 1, 16: time, effective
           GB/s and the fraction of the 8 TB/s HBM peak, with the HBM traffic the
           kernels' FETCH_SIZE / WRITE_SIZE counters read (calibrated on a plain copy)
           when recorded for the current kernel sources
  prefill  the 4-bit codebook workload (3072 x 3072) at M = 2048 and 256: TFLOP/s and the
           fraction of the 2.5 PFLOP/s dense bf16 matrix-core peak, with the matrix-core
           busy fraction and the engine clock from the kernels' counters when recorded
           for the current kernel sources
  roofline the decode kernel of the step (its only kernel) against the HBM peak
  cpu_baseline  the CPU oracle on the same INT4 workload on the host cores, in the two
           reference styles of the OrbitQuant benchmark (dequantise then multiply on
           every call; a weight dequantised once, the product only) and a float32 product
  sweep    (--sweep) MXFP4 at M = 64, INT8 SwiGLU at M = 128, every weight format at the
           codebook prefill's shape, torch's dense bf16 product there (context), the
           grouped (mixture-of-experts) linear, the on-device quantiser, the in-place INT8
           low-rank merge and the INT8-compute (W4A8 / W8A8) linear

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu] [--sweep]
Profiling helpers (used to write the summaries kept with the benchmark):
  python bench.py --probe decode|prefill   counter-collection workloads, no timing
  python bench.py --summarize-trace D [--legs]  per-kernel durations from a rocprofv3 CSV
                                           trace (--legs: per leg of a default run)
  python bench.py --summarize-pmc F W      decode traffic per forward from FETCH_SIZE /
                                           WRITE_SIZE runs of --probe decode
  python bench.py --summarize-prefill P T  matrix-core busy and clock per prefill leg from
                                           a counter run and a trace run of --probe prefill
  python bench.py --summarize-counters P.. any counters of the prefill legs' tile kernel
                                           (stall, LDS, L2 and TA figures) from counter runs
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
POOL_BYTES = 1 << 30           # > 4 x the 256 MB Infinity Cache
FLUSH_BYTES = 1 << 30          # read before every timed replay
AUX_WARM_S = 0.25              # untimed replays before each timed leg
COPY_BYTES = 256 << 20         # calibration copy for the traffic counters
CUS = 256
SIMDS = 1024                   # 256 compute units x 4
XCDS = 8

# decode legs of the default line: (label, workload, M); the step is the INT4 M = 16 leg
DECODE_LEGS = [
    ("int4_asym_g128_4096x4096/M1", "int4_asym_decode", 1),
    ("int4_asym_g128_4096x4096/M4", "int4_asym_decode", 4),
    ("int4_asym_g128_4096x4096/M8", "int4_asym_decode", 8),
    ("int4_asym_g128_4096x4096/M16", "int4_asym_decode", 16),
    ("mxfp4_up_28672x4096/M1", "mxfp4_up", 1),
    ("mxfp4_up_28672x4096/M16", "mxfp4_up", 16),
    ("mxfp4_down_4096x14336/M1", "mxfp4_down", 1),
    ("mxfp4_down_4096x14336/M16", "mxfp4_down", 16),
    ("int8_g256_swiglu_8192x28672/M1", "int8_swiglu", 1),
    ("int8_g256_swiglu_8192x28672/M16", "int8_swiglu", 16),
]
MAIN_LEG = "int4_asym_g128_4096x4096/M16"
PREFILL_LEGS = [
    ("cb4_3072x3072/M2048", "cb4_prefill", 2048),
    ("cb4_3072x3072/M256", "cb4_prefill", 256),
]
# kernels of a forward (names as the traces show them)
FORWARD_KERNELS = ("qgemv_kernel", "qgemm_lds_kernel", "qmm_kernel", "qreduce_kernel", "swiglu_kernel")

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_legs.txt")
PREFILL_COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_prefill_cb4.txt")


def alg_bytes(fmt, M, N, K, G, zeros, swiglu=False, bias=False):
    """Algorithmic bytes of one forward: packed codes + scales (+ zeros) + A + Y (+ bias)."""
    if fmt == "int8":
        w = N * K
    else:
        w = N * K // 2
    if fmt in ("int4", "int8"):
        s = 2 * N * (K // G) + (N * (K // G) // 2 if zeros else 0)
    elif fmt == "mxfp4":
        s = N * (K // 32)
    else:
        s = 2 * N + 64
    a = M * (2 * K if swiglu else K) * 2
    y = M * N * 2
    return w + s + a + y + (2 * N if bias else 0)


def leg_bytes(wl, M):
    return alg_bytes(wl["fmt"], M, wl["N"], wl["K"], wl["group"], not wl.get("symmetric", True),
                     bool(wl.get("swiglu")), wl.get("bias_std") is not None)


def _canonical(fmt, N, K, G, sym, seed):
    import torch

    import synthetic as S
    rng = np.random.default_rng(seed)
    codes, scales, aux = S.random_codes(rng, fmt, N, K, G, symmetric=sym)
    dev = "cuda"
    c = torch.from_numpy(codes).to(dev)
    if fmt == "int4":
        s = torch.from_numpy(scales).to(dev)
        a = None if aux is None else torch.from_numpy(aux).to(dev)
    elif fmt == "mxfp4":
        s = torch.from_numpy(scales).to(dev)
        a = None
    else:
        s = torch.from_numpy(scales.view(np.int16)).to(dev).view(torch.bfloat16)
        a = None
    if fmt == "cb4":
        # a symmetric 16-level codebook (Lloyd-Max levels of N(0,1) to four digits)
        half = np.array([0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733], dtype=np.float32)
        a = np.concatenate([-half[::-1], half]).astype(np.float32)
    return c, s, a


def _pool(Q, fmt, N, K, G, sym, seed, pool_bytes):
    import torch
    c, s, a = _canonical(fmt, N, K, G, sym, seed)
    pw = Q.pack(fmt, N, K, G, c, s, a)
    per = pw.w.numel() + pw.s.numel() + (0 if pw.aux is None else pw.aux.numel())
    n = max(1, int(np.ceil(pool_bytes / per)))
    pool = [pw]
    for _ in range(n - 1):
        pool.append(Q.PackedWeight(pw.fmt, pw.N, pw.K, pw.group, pw.has_zeros, pw.w.clone(), pw.s.clone(),
                                   None if pw.aux is None else pw.aux.clone()))
    torch.cuda.synchronize()
    return pool


def _leg_pool(Q, wl, seed, pool_bytes=POOL_BYTES):
    return _pool(Q, wl["fmt"], wl["N"], wl["K"], wl["group"], wl.get("symmetric", True), seed, pool_bytes)


def kernel_source_hash() -> str:
    """sha256 over every kernel source of the library: a recorded counter figure is
    used only while it matches."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_weight_only_offline_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode())
                h.update(fh.read())
    return h.hexdigest()


def recorded(path):
    """{label: {key: value}} from a counter summary, or {} when it is missing or was
    measured on other kernel sources.  Lines 'leg <label> <key>=<value> ...'."""
    try:
        with open(path) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return {}
    kv = dict(ln.split(":", 1) for ln in lines if ":" in ln and not ln.startswith(("#", " ", "leg ")))
    if kv.get("source_sha256", "").strip() != kernel_source_hash():
        return {}
    out = {}
    for ln in lines:
        if ln.startswith("leg "):
            parts = ln.split()
            out[parts[1]] = {k: float(v) for k, v in (p.split("=", 1) for p in parts[2:] if "=" in p)}
    return out


def _rows(pattern):
    out = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def summarize_trace(d):
    """Per-kernel dispatch count and duration (µs) from a rocprofv3 --kernel-trace CSV."""
    rows = _rows(os.path.join(d, "**", "*kernel_trace.csv"))
    agg = {}
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg.setdefault(r["Kernel_Name"], []).append(dur)
    lines = [f"{'calls':>6} {'avg_us':>9} {'median_us':>9} {'p95_us':>8} {'min_us':>8} {'max_us':>8}  kernel"]
    for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        p95 = v[min(len(v) - 1, int(np.ceil(0.95 * len(v))) - 1)]
        lines.append(f"{len(v):6d} {sum(v) / len(v):9.3f} {v[len(v) // 2]:9.3f} {p95:8.3f} {v[0]:8.3f} {v[-1]:8.3f}  "
                     f"{name}")
    return "\n".join(lines)


def summarize_trace_legs(d):
    """Per-leg kernel durations (µs) from a kernel trace of the default benchmark run,
    split at its marker fills (one before each decode and prefill leg)."""
    rows = _rows(os.path.join(d, "**", "*kernel_trace.csv"))
    segs = _segments(rows)
    labels = [lb for lb, _, _ in DECODE_LEGS] + [lb for lb, _, _ in PREFILL_LEGS]
    if len(segs) < len(labels):
        raise SystemExit(f"{len(segs)} segments, expected {len(labels)} legs")
    lines = [f"{'leg':34s} {'calls':>6} {'avg_us':>9} {'median_us':>9} {'p95_us':>8} {'min_us':>8}  kernel"]
    for label, seg in zip(labels, segs):
        agg = {}
        for g in seg:
            name = g[0]["Kernel_Name"]
            if any(k in name for k in FORWARD_KERNELS):
                agg.setdefault(name, []).append((int(g[0]["End_Timestamp"]) - int(g[0]["Start_Timestamp"])) / 1e3)
        for name, v in agg.items():
            v = sorted(v)
            p95 = v[min(len(v) - 1, int(np.ceil(0.95 * len(v))) - 1)]
            lines.append(f"{label:34s} {len(v):6d} {sum(v) / len(v):9.3f} {v[len(v) // 2]:9.3f} {p95:8.3f} "
                         f"{v[0]:8.3f}  {_short(name)}")
    return "\n".join(lines)


def _short(name):
    """A kernel name without its argument list."""
    return name.replace("(anonymous namespace)", "anon").split("(")[0]


def _segments(rows, key=None):
    """Dispatch rows in dispatch order, split at the probe's marker fills (a torch fill of
    an int32 tensor between legs): [segment][rows]."""
    def did(r):
        return int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
    by = {}
    for r in rows:
        by.setdefault(did(r), []).append(r)
    segs, cur = [], None
    for d in sorted(by):
        name = by[d][0]["Kernel_Name"]
        if "FillFunctor<int>" in name:
            if cur is not None:
                segs.append(cur)
            cur = []
        elif cur is not None:
            cur.append(by[d])
    if cur is not None:
        segs.append(cur)
    return segs


def summarize_pmc(fetch_dir, write_dir):
    """Traffic per forward of every decode leg from a FETCH_SIZE run and a WRITE_SIZE run
    of `bench.py --probe decode`, each counter scaled by what it reads for the plain device
    copy of COPY_BYTES (the first segment of the probe)."""
    res = {}
    for tag, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = [r for r in _rows(os.path.join(d, "**", "*counter_collection.csv")) if r["Counter_Name"] == counter]
        segs = _segments(rows)
        if len(segs) != 1 + len(DECODE_LEGS):
            raise SystemExit(f"{counter}: {len(segs)} segments, expected {1 + len(DECODE_LEGS)}")
        copies = [float(g[0]["Counter_Value"]) for g in segs[0] if "copy" in g[0]["Kernel_Name"].lower()]
        copies = [v for v in copies if v * 1024 > COPY_BYTES / 2]
        if not copies:
            raise SystemExit(f"{counter}: calibration copy not found")
        copy_kib = float(np.median(copies))
        factor = (COPY_BYTES / 1024.0) / copy_kib
        legs = {}
        for (label, _, _), seg in zip(DECODE_LEGS, segs[1:]):
            per_kernel = {}
            for g in seg:
                name = g[0]["Kernel_Name"]
                if any(k in name for k in FORWARD_KERNELS):
                    per_kernel.setdefault(name, []).append(sum(float(r["Counter_Value"]) for r in g))
            legs[label] = dict(kib=sum(float(np.median(v)) for v in per_kernel.values()),
                               kernels={k: len(v) for k, v in per_kernel.items()})
        res[tag] = dict(copy_kib=copy_kib, factor=factor, legs=legs)
    lines = []
    for tag in ("fetch", "write"):
        lines.append(f"{tag}: calibration copy {res[tag]['copy_kib']:.1f} KiB per dispatch for {COPY_BYTES // 1024} KiB "
                     f"copied -> factor {res[tag]['factor']:.4f}")
    import synthetic as S
    for label, wname, M in DECODE_LEGS:
        wl = S.WORKLOADS[wname]
        f = res["fetch"]["legs"][label]
        w = res["write"]["legs"][label]
        fb = f["kib"] * 1024 * res["fetch"]["factor"]
        wb = w["kib"] * 1024 * res["write"]["factor"]
        ab = leg_bytes(wl, M)
        kern = ";".join(f"{_short(k)} x{n}" for k, n in f["kernels"].items())
        lines.append(f"leg {label} fetch_bytes={fb:.0f} write_bytes={wb:.0f} traffic_bytes={fb + wb:.0f} "
                     f"alg_bytes={ab} ratio={(fb + wb) / ab:.4f}")
        lines.append(f"  kernels of {label}: {kern}")
    lines.append(f"source_sha256: {kernel_source_hash()}")
    return "\n".join(lines)


def summarize_prefill(pmc_dir, trace_dir):
    """Matrix-core busy fraction, engine clock and instruction mix per prefill leg from a
    counter run and a trace run of `bench.py --probe prefill`."""
    rows = _rows(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    segs = _segments(rows)
    trows = _rows(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    tsegs = _segments(trows)
    if len(segs) != len(PREFILL_LEGS) or len(tsegs) != len(PREFILL_LEGS):
        raise SystemExit(f"{len(segs)} / {len(tsegs)} segments, expected {len(PREFILL_LEGS)}")
    lines = []
    for (label, _, M), seg, tseg in zip(PREFILL_LEGS, segs, tsegs):
        main = [g for g in seg if "qgemm_lds_kernel" in g[0]["Kernel_Name"] or "qmm_kernel" in g[0]["Kernel_Name"]]
        if not main:
            raise SystemExit(f"{label}: no tile kernel dispatches")
        cnt = {}
        for g in main:
            per = {}
            for r in g:
                per[r["Counter_Name"]] = per.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            for k, v in per.items():
                cnt.setdefault(k, []).append(v)
        med = {k: float(np.median(v)) for k, v in cnt.items()}
        durs = sorted((int(g[0]["End_Timestamp"]) - int(g[0]["Start_Timestamp"])) / 1e3 for g in tseg
                      if "qgemm_lds_kernel" in g[0]["Kernel_Name"] or "qmm_kernel" in g[0]["Kernel_Name"])
        us = durs[len(durs) // 2]
        cycles = med["GRBM_GUI_ACTIVE"] / XCDS
        busy = med["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / cycles
        # engine clock: the GPU-busy cycles of the counter run over the kernel's traced
        # duration (another run); the busy count also covers the dispatch around the
        # kernel, so only kernels of 30 us and more give a usable figure
        ghz = f" clock_ghz={cycles / (us * 1e3):.3f}" if us >= 30.0 else ""
        lines.append(f"leg {label} mfma_busy={busy:.4f}{ghz} kernel_us={us:.3f} "
                     f"mfma_insts={med['SQ_INSTS_MFMA']:.0f} valu_per_mfma={(med['SQ_INSTS_VALU'] - med['SQ_INSTS_MFMA']) / med['SQ_INSTS_MFMA']:.3f} "
                     f"lds_insts={med['SQ_INSTS_LDS']:.0f} lds_bank_conflict_cycles={med['SQ_LDS_BANK_CONFLICT']:.0f}")
        lines.append(f"  kernel of {label}: {_short(main[0][0]['Kernel_Name'])} ({len(main)} dispatches)")
    lines.append(f"source_sha256: {kernel_source_hash()}")
    return "\n".join(lines)



def summarize_counters(*pmc_dirs):
    """Where the tile kernel of each prefill leg spends its time, from counter runs of
    `bench.py --probe prefill` (any counters, one or more runs): the median per dispatch of
    every counter, and the fractions derived from those present.  SQ wave-cycle counters
    count quad-cycles summed over waves; SIMD- and CU-cycle counters are per SIMD / CU."""
    lines = []
    med = {}
    for d in pmc_dirs:
        segs = _segments(_rows(os.path.join(d, "**", "*counter_collection.csv")))
        if len(segs) != len(PREFILL_LEGS):
            raise SystemExit(f"{d}: {len(segs)} segments, expected {len(PREFILL_LEGS)}")
        for (label, _, _), seg in zip(PREFILL_LEGS, segs):
            main = [g for g in seg if "qgemm_lds_kernel" in g[0]["Kernel_Name"]]
            cnt = {}
            for g in main:
                per = {}
                for r in g:
                    per[r["Counter_Name"]] = per.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                for k, v in per.items():
                    cnt.setdefault(k, []).append(v)
            m = med.setdefault(label, {"kernel": _short(main[0][0]["Kernel_Name"]) if main else ""})
            for k, v in cnt.items():
                m[f"{k}@{os.path.basename(os.path.normpath(d))}"] = float(np.median(v))
    for label, m in med.items():
        lines.append(f"tile kernel of {label}: {m.pop('kernel')}")
        def get(name):
            vals = [v for k, v in m.items() if k.split("@")[0] == name]
            return vals[0] if vals else None
        for k in sorted(m):
            lines.append(f"   {k:48s} {m[k]:16.1f}")
        wave, cyc = get("SQ_WAVE_CYCLES"), get("GRBM_GUI_ACTIVE")
        derived = []
        if wave:
            for name in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                         "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS"):
                if get(name) is not None:
                    derived.append(f"{name.lower()[3:]}/wave_cycles={get(name) / wave:.3f}")
        if cyc:
            c = cyc / XCDS
            if get("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
                derived.append(f"mfma_busy={get('SQ_VALU_MFMA_BUSY_CYCLES') / SIMDS / c:.3f}")
            if get("SQ_VALU_MFMA_COEXEC_CYCLES") is not None:
                derived.append(f"valu_coexec_with_mfma={get('SQ_VALU_MFMA_COEXEC_CYCLES') / SIMDS / c:.3f}")
            if get("SQ_LDS_IDX_ACTIVE") is not None:
                derived.append(f"lds_busy={get('SQ_LDS_IDX_ACTIVE') / CUS / c:.3f}")
            if get("TA_TA_BUSY") is not None:
                derived.append(f"ta_busy={get('TA_TA_BUSY') / CUS / c:.3f}")
        if get("TCC_HIT") is not None and get("TCC_MISS") is not None:
            derived.append(f"l2_hit={get('TCC_HIT') / (get('TCC_HIT') + get('TCC_MISS')):.3f}")
        lines.append("   derived: " + " ".join(derived))
    lines.append(f"source_sha256: {kernel_source_hash()}")
    return "\n".join(lines)

class Flush:
    """Reads FLUSH_BYTES of device memory (four times the Infinity Cache), so that a
    following forward finds nothing of its working set cached.  A max-reduction over
    int32 reads the buffer and writes one value: a sum would first widen it to int64 (a
    2 GiB write), and the caches would then hold dirty lines that the timed forwards
    pay to write back.  Queued without a wait: the GPU is still busy with it while the
    host queues the timed work behind it."""

    def __init__(self):
        import torch
        # filled as bytes (a uint8 fill, not the int32 fill that marks legs in a trace)
        self.buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda").view(torch.int32)
        self.sink = None

    def __call__(self):
        self.sink = self.buf.amax()


def time_forward(Q, pool, x, act, steps, warmup, flush, use_graph=True, schedule=None, warm_s=0.0, reps=1):
    """Average time (ms) of one forward over `steps` forwards, forward i on pool copy
    i mod len(pool).

    With a graph: one untimed replay, more untimed replays until warm_s seconds have
    passed (so the clocks have settled under this load), then `reps` timed replays of
    the `steps` forwards, each right behind a cache flush; the median replay is returned."""
    import torch
    pw0 = pool[0]
    M = x.shape[0]
    out = torch.empty((M, pw0.N), dtype=torch.bfloat16, device=x.device)
    wsb = Q.workspace_bytes(pw0.fmt, M, pw0.N, pw0.K, pw0.group, act, schedule)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=x.device)

    def run(i):
        Q.linear(x, pool[i % len(pool)], act=act, out=out, workspace=ws, schedule=schedule)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    times = []
    if use_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(steps):
                    run(i)
        torch.cuda.synchronize()
        g.replay()                     # warm replay
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            g.replay()
            torch.cuda.synchronize()
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            flush()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / steps)
        del g
    else:
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            flush()
            e0.record()
            for i in range(steps):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / steps)
    return sorted(times)[len(times) // 2], out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl_name, M, seconds=2.5, runs=3):
    """The oracle as it stands on host cores, on the INT4 decode workload at M rows:
    (i) dequantise then the float64 product on every call (the oracle's forward), the
    reported value; (ii) the weight dequantised once, the float64 product only; (iii) the
    same product in float32.  Each style: `runs` runs of about `seconds` each, the median."""
    import oracle as O
    import synthetic as S
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    wl = S.WORKLOADS[wl_name]
    N, K, G = wl["N"], wl["K"], wl["group"]
    canon = O.quantize("int4", S.weights(wl), G, symmetric=wl["symmetric"])
    x = S.activations(wl, M)
    dw = O.dequant("int4", canon, K)
    x32 = np.asarray(x, dtype=np.float32)
    styles = {
        "dequantize_then_linear_f64": lambda: O.forward("int4", x, canon, K),
        "predequantized_f64": lambda: O.linear_ref(x, dw),
        "predequantized_f32": lambda: x32 @ dw.T,
    }
    b = alg_bytes("int4", M, N, K, G, not wl["symmetric"])
    res = {}
    for name, fn in styles.items():
        per = []
        for _ in range(runs):
            n, t0 = 0, time.perf_counter()
            while True:
                fn()
                n += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            per.append((time.perf_counter() - t0) / n)
        dt = statistics.median(per)
        res[name] = {"ms": round(dt * 1e3, 3), "GB/s": round(b / dt / 1e9, 4)}
    main = res["dequantize_then_linear_f64"]
    return {"value": main["GB/s"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the {N}x{K} INT4 weight (zero-points, g128) at M={M}: median of {runs} runs of "
                      f"~{seconds:g} s per style; value = dequantise + float64 product per call",
            "styles": res, "cpu_model": _cpu_model(), "nproc": len(os.sched_getaffinity(0))}


def probe(which="decode"):
    """Counter-collection workloads, no timing; legs are separated by a marker fill.
    decode: a plain device copy of COPY_BYTES three times (the calibration of FETCH_SIZE /
    WRITE_SIZE), then 20 forwards of each decode leg; prefill: 20 forwards of each
    prefill leg.  Each forward reads the next copy of a 1 GiB weight pool."""
    import torch

    import bit_weight_only_offline_amd as Q
    import synthetic as S
    torch.cuda.set_device(0)
    marker = torch.empty(1, dtype=torch.int32, device="cuda")
    legs = DECODE_LEGS if which == "decode" else PREFILL_LEGS
    if which == "decode":
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        marker.fill_(0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    pools = {}
    for i, (label, wname, M) in enumerate(legs):
        wl = S.WORKLOADS[wname]
        if wname not in pools:
            pools.clear()
            torch.cuda.empty_cache()
            pools[wname] = _leg_pool(Q, wl, 7)
        pool = pools[wname]
        x = torch.from_numpy(S.activations(wl, M)).cuda().to(torch.bfloat16)
        act = "swiglu" if wl.get("swiglu") else None
        out = torch.empty((M, wl["N"]), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(Q.workspace_bytes(wl["fmt"], M, wl["N"], wl["K"], wl["group"], act), 256),
                         dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        marker.fill_(i + 1)
        for j in range(20):
            Q.linear(x, pool[j % len(pool)], act=act, out=out, workspace=ws)
        torch.cuda.synchronize()
        print(f"probe: {label} x20 ({Q.default_schedule(wl['fmt'], M, wl['N'], wl['K'], wl['group'], act)})",
              flush=True)
    print(f"probe: done (kernel sources sha256 {kernel_source_hash()})", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also the sweep workloads (see the module docstring)")
    ap.add_argument("--cpu-seconds", type=float, default=2.5, help="seconds per CPU-baseline run (3 runs per style)")
    ap.add_argument("--probe", choices=("decode", "prefill"))
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--legs", action="store_true", help="with --summarize-trace: per leg of the default line")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-prefill", nargs=2, metavar=("PMC_DIR", "TRACE_DIR"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace_legs(args.summarize_trace) if args.legs else summarize_trace(args.summarize_trace))
        return
    if args.summarize_pmc:
        print(summarize_pmc(*args.summarize_pmc))
        return
    if args.summarize_prefill:
        print(summarize_prefill(*args.summarize_prefill))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU (it has no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.probe:
        probe(args.probe)
        return

    import torch

    import bit_weight_only_offline_amd as Q
    import synthetic as S
    torch.cuda.set_device(0)
    use_graph = not args.no_graph
    flush = Flush()
    traffic = recorded(TRAFFIC_FILE)
    pcount = recorded(PREFILL_COUNTERS_FILE)
    # a marker fill before each leg, so that a kernel trace of this run splits per leg
    # (bench.py --summarize-trace D --legs); outside every timed region
    marker = torch.empty(1, dtype=torch.int32, device="cuda")
    leg_no = [0]

    def mark():
        marker.fill_(leg_no[0])
        leg_no[0] += 1

    # ---- decode legs; the step is the INT4 zero-point decode at M = 16 ----
    decode = {}
    main_ms = main_copies = None
    pool, pool_name = None, None
    for label, wname, M in DECODE_LEGS:
        wl = S.WORKLOADS[wname]
        if pool_name != wname:
            pool = None
            torch.cuda.empty_cache()
            pool, pool_name = _leg_pool(Q, wl, 7), wname
        x = torch.from_numpy(S.activations(wl, M)).cuda().to(torch.bfloat16)
        act = "swiglu" if wl.get("swiglu") else None
        mark()
        if label == MAIN_LEG:
            # exactly --steps forwards per timed replay, one timed replay
            ms, _ = time_forward(Q, pool, x, act, args.steps, args.warmup, flush, use_graph, warm_s=AUX_WARM_S)
            main_ms, main_copies = ms, len(pool)
        else:
            ms, _ = time_forward(Q, pool, x, act, max(20, len(pool)), 5, flush, use_graph, warm_s=AUX_WARM_S, reps=3)
        b = leg_bytes(wl, M)
        gbs = b / (ms * 1e-3) / 1e9
        sch = Q.default_schedule(wl["fmt"], M, wl["N"], wl["K"], wl["group"], act)
        decode[label] = {"us": round(ms * 1e3, 3), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "alg_bytes": b, "traffic": (int(traffic[label]["traffic_bytes"]) if label in traffic else None),
                         "schedule": f"tile {sch.tile}, splits {sch.splits}"}
    pool = None
    torch.cuda.empty_cache()
    main_leg = decode[MAIN_LEG]
    value = main_leg["GB/s"]

    # ---- prefill legs: the codebook workload ----
    prefill = {}
    for label, wname, M in PREFILL_LEGS:
        wl = S.WORKLOADS[wname]
        if pool_name != wname:
            pool = None
            torch.cuda.empty_cache()
            pool, pool_name = _leg_pool(Q, wl, 5), wname
        x = torch.from_numpy(S.activations(wl, M)).cuda().to(torch.bfloat16)
        mark()
        ms, _ = time_forward(Q, pool, x, None, max(20, len(pool)), 3, flush, use_graph, warm_s=AUX_WARM_S, reps=3)
        fl = 2.0 * M * wl["N"] * wl["K"]
        tf = fl / (ms * 1e-3) / 1e12
        sch = Q.default_schedule(wl["fmt"], M, wl["N"], wl["K"], wl["group"])
        c = pcount.get(label, {})
        prefill[label] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
                          "mfma_busy_counter": c.get("mfma_busy"), "clock_ghz_counter": c.get("clock_ghz"),
                          "schedule": f"tile {sch.tile}, splits {sch.splits}"}
    pool = None
    torch.cuda.empty_cache()
    mark()                                  # end of the legs of the line

    use_graph_sweep = use_graph
    others = {}
    if args.sweep:
        for name, M_list in (("mxfp4_up", (64,)), ("mxfp4_down", (64,)), ("int8_swiglu", (128,))):
            w_ = S.WORKLOADS[name]
            fmt = w_["fmt"]
            pl = _pool(Q, fmt, w_["N"], w_["K"], w_["group"], True, 7, POOL_BYTES)
            for M in M_list:
                xa = torch.from_numpy(S.activations(w_, M)).cuda().to(torch.bfloat16)
                act = "swiglu" if w_.get("swiglu") else None
                ms, _ = time_forward(Q, pl, xa, act, max(20, len(pl)), 5, flush, use_graph_sweep, warm_s=AUX_WARM_S, reps=3)
                b = alg_bytes(fmt, M, w_["N"], w_["K"], w_["group"], False, bool(act), w_.get("bias_std") is not None)
                fl = 2.0 * M * w_["N"] * w_["K"]
                others[f"{name}/M{M}"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                                          "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1)}
            del pl
            torch.cuda.empty_cache()
        # the other weight formats at the codebook prefill's shape (3072 x 3072, M = 2048),
        # default schedules, weights from a pool as above
        wl5 = S.WORKLOADS["cb4_prefill"]
        xp = torch.from_numpy(S.activations(wl5, 2048)).cuda().to(torch.bfloat16)
        for fmt, Gf, sym in (("int4", 128, True), ("int4", 128, False), ("mxfp4", 32, True), ("int8", 256, True)):
            pl = _pool(Q, fmt, wl5["N"], wl5["K"], Gf, sym, 8, POOL_BYTES)
            ms, _ = time_forward(Q, pl, xp, None, max(20, len(pl)), 5, flush, use_graph_sweep, warm_s=AUX_WARM_S, reps=3)
            fl = 2.0 * 2048 * wl5["N"] * wl5["K"]
            tf = fl / (ms * 1e-3) / 1e12
            others[f"{fmt}{'' if sym else '_asym'}_g{Gf}_3072/M2048"] = {
                "us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
            del pl
            torch.cuda.empty_cache()
        # context, not this library: torch's dense bf16 product (hipBLASLt) at the same
        # shape, a pool of contiguous [K, N] weights cycled like the packed ones
        wt = torch.randn(wl5["K"], wl5["N"], device="cuda").to(torch.bfloat16)
        dense = [wt] + [wt.clone() for _ in range(max(0, int(np.ceil(POOL_BYTES / (wt.numel() * 2))) - 1))]
        yd = torch.empty((2048, wl5["N"]), dtype=torch.bfloat16, device="cuda")
        steps_d = max(20, len(dense))
        for i in range(5):
            torch.matmul(xp, dense[i % len(dense)], out=yd)
        torch.cuda.synchronize()
        gd, sd = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        sd.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sd):
            with torch.cuda.graph(gd, stream=sd):
                for i in range(steps_d):
                    torch.matmul(xp, dense[i % len(dense)], out=yd)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < AUX_WARM_S:
            gd.replay()
            torch.cuda.synchronize()
        tds = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gd.replay()
            e1.record()
            torch.cuda.synchronize()
            tds.append(e0.elapsed_time(e1) / steps_d)
        msd = sorted(tds)[1]
        fl = 2.0 * 2048 * wl5["N"] * wl5["K"]
        others["torch_bf16_matmul_3072/M2048"] = {"us": round(msd * 1e3, 2), "TFLOP/s": round(fl / (msd * 1e-3) / 1e12, 1),
                                                  "mfma_frac": round(fl / (msd * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del gd, dense, wt, yd
        torch.cuda.empty_cache()
        del xp

    moe = {}
    if args.sweep:
        # mixture of experts: eight MXFP4 experts of the down projection (4096 x 14336),
        # tokens routed uniformly at random (seeded); weights of the used experts from HBM
        E, N_, K_ = 8, 4096, 14336
        rng = np.random.default_rng(12)
        c, s_, _ = _canonical("mxfp4", N_, K_, 32, True, 12)
        pe = Q.pack_experts("mxfp4", N_, K_, 32, [(c, s_, None)] * E)
        per_e = pe.w.numel() // E + pe.s.numel() // E
        copies = max(1, int(np.ceil(POOL_BYTES / (per_e * E))))
        pes = [pe] + [Q.PackedExperts(pe.fmt, E, N_, K_, 32, 0, pe.w.clone(), pe.s.clone(), None)
                      for _ in range(copies - 1)]
        for T in (16, 256):
            cnt = np.bincount(rng.integers(0, E, T), minlength=E).astype(np.int32)
            cnt_t = torch.from_numpy(cnt).cuda()
            xm = torch.from_numpy(S.to_bf16_values(rng.standard_normal((T, K_)).astype(np.float32))).cuda().to(
                torch.bfloat16)
            outm = torch.empty((T, N_), dtype=torch.bfloat16, device="cuda")
            wsm = torch.zeros(max(Q.grouped_workspace_bytes("mxfp4", T, E, N_, K_, 32), 256), dtype=torch.uint8,
                              device="cuda")

            def run_moe(i):
                Q.grouped_linear(xm, pes[i % len(pes)], cnt_t, out=outm, workspace=wsm)

            for i in range(5):
                run_moe(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            steps = 40
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    for i in range(steps):
                        run_moe(i)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            used = int((cnt > 0).sum())
            nb = used * per_e + T * K_ * 2 + T * N_ * 2
            moe[f"mxfp4_down_E8/T{T}"] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                                          "experts_used": used}
            del g
        del pes, pe
        torch.cuda.empty_cache()

    quant = {}
    if args.sweep:
        # on-device quantiser: dense float32 weights -> canonical codes and scales
        for name in ("mxfp4_up", "int8_swiglu", "int4_asym_decode", "cb4_prefill"):
            w_ = S.WORKLOADS[name]
            fmt = w_["fmt"]
            wd = torch.from_numpy(S.weights(w_)).cuda()
            lv = None
            if fmt == "cb4":
                half = np.array([0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733], dtype=np.float32)
                lv = np.concatenate([-half[::-1], half]).astype(np.float32)
            sym = w_.get("symmetric", True)
            for _ in range(3):
                Q.quantize(fmt, wd, w_["group"], symmetric=sym, levels=lv)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                Q.quantize(fmt, wd, w_["group"], symmetric=sym, levels=lv)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            nb = wd.numel() * 4 + (wd.numel() if fmt == "int8" else wd.numel() // 2)   # fp32 in + codes out
            quant[name] = {"us": round(ms * 1e3, 1), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1)}
            del wd
            torch.cuda.empty_cache()

    a8 = {}
    if args.sweep:
        # INT8-compute path (W4A8 / W8A8) at the prefill shape 3072 x 3072: default
        # schedule, activation quantisation included, weights from HBM
        for fmt_, G_ in (("int4", 128), ("int8", 128)):
            pl = _pool(Q, fmt_, 3072, 3072, G_, True, 17, POOL_BYTES)
            for M in (256, 2048):
                xa = torch.randn(M, 3072, device="cuda").to(torch.bfloat16)
                outa = torch.empty(M, 3072, device="cuda", dtype=torch.bfloat16)
                wsa = torch.empty(Q.a8_workspace_bytes(fmt_, M, 3072, 3072, G_) + 256, dtype=torch.uint8,
                                  device="cuda")
                n_a8 = max(40, len(pl))      # every pool copy once: weights from HBM
                t0 = time.perf_counter()
                while True:
                    for i in range(n_a8):
                        Q.linear_a8(xa, pl[i % len(pl)], out=outa, workspace=wsa)
                    torch.cuda.synchronize()
                    if time.perf_counter() - t0 >= AUX_WARM_S:
                        break
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(n_a8):
                    Q.linear_a8(xa, pl[i % len(pl)], out=outa, workspace=wsa)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / n_a8
                a8[f"{fmt_}_g{G_}_3072/M{M}"] = {"us": round(ms * 1e3, 2),
                                                 "TOPS": round(2.0 * M * 3072 * 3072 / (ms * 1e-3) / 1e12, 1)}
            del pl
            torch.cuda.empty_cache()

    merge = {}
    if args.sweep:
        # in-place INT8 low-rank merge on the INT8 SwiGLU layer's weight (8192 x 28672,
        # group 256), rank 16 and 64, nearest and stochastic rounding
        w_ = S.WORKLOADS["int8_swiglu"]
        N_, K_, G_ = w_["N"], w_["K"], w_["group"]
        rng = np.random.default_rng(31)
        pw = Q.pack("int8", N_, K_, G_, *_canonical("int8", N_, K_, G_, True, 31))
        for r in (16, 64):
            a = torch.from_numpy(S.to_bf16_values((rng.standard_normal((N_, r)) * 1e-3).astype(np.float32))).cuda()
            b = torch.from_numpy(S.to_bf16_values((rng.standard_normal((r, K_)) * 1e-3).astype(np.float32))).cuda()
            a, b = a.to(torch.bfloat16), b.to(torch.bfloat16)
            for seed in (None, 1):
                for _ in range(2):
                    Q.int8_addmm_(pw, a, b, alpha=1.0, rounding_seed=seed)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(5):
                    Q.int8_addmm_(pw, a, b, alpha=1.0, rounding_seed=seed)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 5
                nb = 2 * N_ * K_ + 4 * N_ * (K_ // G_) + 2 * r * (N_ + K_)    # codes and scales read and written
                merge[f"r{r}/{'nearest' if seed is None else 'stochastic'}"] = {
                    "us": round(ms * 1e3, 1), "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                    "GFLOP/s": round(2.0 * N_ * K_ * r / (ms * 1e-3) / 1e9, 1)}
        del pw
        torch.cuda.empty_cache()


    cpu = None if args.no_cpu else cpu_baseline("int4_asym_decode", 16, args.cpu_seconds)
    wl2 = S.WORKLOADS["int4_asym_decode"]
    rec = {
        "metric": "W4A16 linear: effective HBM GB/s at M=1-16; TFLOP/s + MFMA util at M=2048",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "int4 asym g128 decode linear, W 4096x4096 (fp16 scales, 4-bit zeros), "
                               "X bf16 [16,4096], bf16 out", "M": 16, "N": wl2["N"], "K": wl2["K"],
                   "group": wl2["group"], "weight_pool_copies": main_copies, "hip_graph": use_graph,
                   "cache": "1 GiB read before the timed replay", "schedule": main_leg["schedule"]},
        "roofline": {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": main_leg["traffic"],
                     "kernel": "qgemv_kernel (INT4, zero-points, group 128)", "alg_bytes": main_leg["alg_bytes"],
                     "us_per_launch": main_leg["us"]},
        "decode": decode,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    if others:
        rec["others"] = others
    if quant:
        rec["quantize"] = quant
    if merge:
        rec["int8_merge"] = merge
    if a8:
        rec["int8_compute"] = a8
    if moe:
        rec["moe"] = moe
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
