"""Benchmark of the weight-only low-bit linear layer on one MI355X.

One step = one forward of the INT4 decode workload with zero-points (group 128, fp16
scales, 4-bit zeros): X bf16 [16, 4096] times a packed 4096 x 4096 weight, bf16 out.
The metric is effective HBM bandwidth: algorithmic bytes (packed weight + scales +
zero-points + X + Y) per step over the step time.  Each step reads a different copy
of the packed weight from a pool larger than twice the 256 MB Infinity Cache, so the
weights come from HBM.  Steps run back to back inside a HIP graph (the launch-bound
inner loop), timed with HIP events on the stream the kernels run on.

Also reported, on the same line:
  prefill  the 4-bit codebook workload at M = 2048 (3072 x 3072): TFLOP/s and the
           fraction of the dense bf16 matrix-core peak
  roofline the decode kernel (the only kernel of the step) against the HBM peak
           (8 TB/s), with the HBM traffic its FETCH_SIZE / WRITE_SIZE counters read
           (calibrated on a plain copy), when recorded for the current kernel source
  cpu_baseline  the CPU oracle (dequantise, then a float64 product) on a bounded
           sample of the same workload, on the host cores
  sweep    (--sweep) the decode workload at M = 1, 4, 8, the other workloads, the grouped
           (mixture-of-experts) linear, the on-device quantiser (float32 weights in,
           canonical codes out), the in-place INT8 low-rank merge and the INT8-compute
           (W4A8 / W8A8) linear

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu] [--sweep]
Profiling helpers (used to write the summaries kept with the benchmark):
  python bench.py --probe [decode|prefill]   copy calibration + 20 decode dispatches, or
                                       20 prefill dispatches; no timing
  python bench.py --summarize-trace D  per-kernel durations from a rocprofv3 CSV trace
  python bench.py --summarize-pmc F W  traffic per dispatch from FETCH_SIZE / WRITE_SIZE runs
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
POOL_BYTES = 1 << 30           # > 2 x the 256 MB Infinity Cache
AUX_WARM_S = 0.25              # untimed replays before each timed leg after the main step
COPY_BYTES = 256 << 20         # calibration copy for the traffic counters

# sources that define the decode kernel the roofline reports on; a recorded traffic
# figure is used only while their hash is the one it was measured with
KERNEL_SOURCES = ["ql_gemv.hpp", "ql_decode.hpp", "ql_common.hpp", "ql_gemm_dispatch.hpp", "ql_gemm_int4.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qgemv_int4_asym_decode_m16.txt")
DECODE_KERNEL = "qgemv_kernel<0, true, 4"     # prefix of the INT4 zero-point g128 instantiation


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


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_weight_only_offline_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per decode launch recorded in the counter summary, or None when the
    summary is missing or was measured on another version of the kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split(":", 1) for line in fh if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    if kv.get("source_sha256", "").strip() != kernel_source_hash():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


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


def summarize_pmc(fetch_dir, write_dir):
    """Traffic of the decode kernel per dispatch from a FETCH_SIZE run and a WRITE_SIZE
    run of `bench.py --probe`, each scaled by what the counter reads for the plain
    device copy of COPY_BYTES in the same run."""
    def per_kernel(d, counter):
        agg = {}
        for r in _rows(os.path.join(d, "**", "*counter_collection.csv")):
            if r["Counter_Name"] == counter:
                agg.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return agg

    def pick(agg, key):
        vals = [v for k, vs in agg.items() if key in k for v in vs]
        return vals

    out = {}
    for tag, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        agg = per_kernel(d, counter)
        # the calibration copy: the dispatches that moved about COPY_BYTES
        copies = [v for k, vs in agg.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs
                  if v * 1024 > COPY_BYTES / 2]
        kern = pick(agg, DECODE_KERNEL)
        if not copies or not kern:
            raise SystemExit(f"{counter}: calibration copy or decode kernel not found in {d}")
        copy_kib = float(np.median(copies))
        factor = (COPY_BYTES / 1024.0) / copy_kib
        out[tag] = dict(copy_kib=copy_kib, factor=factor, kernel_kib=float(np.median(kern)), n=len(kern))
    traffic = out["fetch"]["kernel_kib"] * 1024 * out["fetch"]["factor"] + \
        out["write"]["kernel_kib"] * 1024 * out["write"]["factor"]
    return out, int(round(traffic))


def time_forward(Q, pool, x, act, steps, warmup, use_graph=True, schedule=None, warm_s=0.0, reps=1):
    """Average time (ms) of one forward over `steps` forwards, each on the next pool copy.

    With a graph: one untimed replay, then more untimed replays until warm_s seconds have
    passed (so the clocks have settled under this load), then `reps` timed replays of the
    `steps` forwards; the median replay is returned."""
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
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / steps)
        ms = sorted(times)[len(times) // 2]
        del g
    else:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
    return ms, out


def cpu_baseline(wl_name, M, seconds=10.0):
    """The oracle as it stands (dequantise, then the float64 product) on host cores."""
    import oracle as O
    import synthetic as S
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    wl = S.WORKLOADS[wl_name]
    N, K, G = wl["N"], wl["K"], wl["group"]
    w = S.weights(wl)
    canon = O.quantize("int4", w, G, symmetric=wl["symmetric"])
    x = S.activations(wl, M)
    t0 = time.perf_counter()
    n = 0
    while True:
        O.forward("int4", x, canon, K)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    b = alg_bytes("int4", M, N, K, G, not wl["symmetric"])
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} full forwards (dequantise + float64 product) of the {N}x{K} INT4 weight at M={M}, "
                      f"{dt * 1e3:.1f} ms each"}


def probe(which="decode"):
    """Counter-collection workload, no timing.  decode: a plain device copy of COPY_BYTES
    (the calibration of FETCH_SIZE / WRITE_SIZE) and 20 dispatches of the decode step;
    prefill: 20 dispatches of the codebook prefill (M = 2048)."""
    import torch

    import bit_weight_only_offline_amd as Q
    import synthetic as S
    torch.cuda.set_device(0)
    if which == "prefill":
        wl5 = S.WORKLOADS["cb4_prefill"]
        pool5 = _pool(Q, "cb4", wl5["N"], wl5["K"], 0, True, 5, 256 << 20)
        x5 = torch.from_numpy(S.activations(wl5, 2048)).cuda().to(torch.bfloat16)
        out = torch.empty((2048, wl5["N"]), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(Q.workspace_bytes("cb4", 2048, wl5["N"], wl5["K"], 0), 256), dtype=torch.uint8,
                         device="cuda")
        for i in range(20):
            Q.linear(x5, pool5[i % len(pool5)], out=out, workspace=ws)
        torch.cuda.synchronize()
        print(f"probe: codebook prefill M=2048 x20 ({Q.default_schedule('cb4', 2048, wl5['N'], wl5['K'], 0)})",
              flush=True)
        return
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    wl = S.WORKLOADS["int4_asym_decode"]
    N, K, G = wl["N"], wl["K"], wl["group"]
    pool = _pool(Q, "int4", N, K, G, False, 2, POOL_BYTES)
    x = torch.from_numpy(S.activations(wl, 16)).cuda().to(torch.bfloat16)
    out = torch.empty((16, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    for i in range(20):
        Q.linear(x, pool[i % len(pool)], out=out, workspace=ws)
    torch.cuda.synchronize()
    print(f"probe: copy {COPY_BYTES} bytes x3, decode M=16 x20 "
          f"(kernel sources sha256 {kernel_source_hash()})", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also M = 1, 4, 8 and every other workload shape")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--probe", nargs="?", const="decode", choices=("decode", "prefill"))
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_pmc:
        parts, traffic = summarize_pmc(*args.summarize_pmc)
        for tag, v in parts.items():
            print(f"{tag}: copy_kib_per_dispatch: {v['copy_kib']:.1f} (copied {COPY_BYTES // 1024} KiB), "
                  f"factor {v['factor']:.4f}; decode_kib_per_dispatch (median of {v['n']}): {v['kernel_kib']:.1f}")
        print(f"source_sha256: {kernel_source_hash()}")
        print(f"traffic_bytes_per_launch: {traffic}")
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

    # ---- the step: INT4 zero-point decode, M = 16 ----
    wl = S.WORKLOADS["int4_asym_decode"]
    N, K, G = wl["N"], wl["K"], wl["group"]
    pool = _pool(Q, "int4", N, K, G, False, 2, POOL_BYTES)
    n_copies = len(pool)
    xs = S.activations(wl, 16)
    x16 = torch.from_numpy(xs[:16]).cuda().to(torch.bfloat16)
    sched = Q.default_schedule("int4", 16, N, K, G)
    main_ms, _ = time_forward(Q, pool, x16, None, args.steps, args.warmup, use_graph)
    b16 = alg_bytes("int4", 16, N, K, G, True)
    value = b16 / (main_ms * 1e-3) / 1e9
    sweep = {}
    if args.sweep:
        for M in (1, 4, 8):
            x = torch.from_numpy(xs[:M]).cuda().to(torch.bfloat16)
            ms, _ = time_forward(Q, pool, x, None, max(50, args.steps // 2), args.warmup, use_graph)
            b = alg_bytes("int4", M, N, K, G, True)
            sweep[str(M)] = {"us": round(ms * 1e3, 3), "GB/s": round(b / (ms * 1e-3) / 1e9, 1)}
        sweep["16"] = {"us": round(main_ms * 1e3, 3), "GB/s": round(value, 1)}
    del pool
    torch.cuda.empty_cache()

    # ---- prefill: 4-bit codebook, 3072 x 3072, M = 2048 ----
    wl5 = S.WORKLOADS["cb4_prefill"]
    # every forward reads the next copy of a 1 GiB pool, all copies once per replay, so the
    # weights come from HBM, not from the Infinity Cache
    pool5 = _pool(Q, "cb4", wl5["N"], wl5["K"], 0, True, 5, POOL_BYTES)
    x5 = torch.from_numpy(S.activations(wl5, 2048)).cuda().to(torch.bfloat16)
    ms5, _ = time_forward(Q, pool5, x5, None, max(len(pool5), args.steps // 4), max(3, args.warmup // 4), use_graph,
                          warm_s=AUX_WARM_S, reps=3)
    fl = 2.0 * 2048 * wl5["N"] * wl5["K"]
    tflops = fl / (ms5 * 1e-3) / 1e12
    prefill = {"workload": "cb4 Lloyd-Max codebook 3072x3072, M=2048, bf16", "us": round(ms5 * 1e3, 2),
               "TFLOP/s": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
               "schedule": repr(Q.default_schedule("cb4", 2048, wl5["N"], wl5["K"], 0))}
    del pool5
    torch.cuda.empty_cache()

    others = {}
    if args.sweep:
        for name, M_list in (("mxfp4_up", (1, 16, 64)), ("mxfp4_down", (1, 16, 64)), ("int8_swiglu", (1, 16, 128)),
                             ("cb4_prefill", (256,))):
            w_ = S.WORKLOADS[name]
            fmt = w_["fmt"]
            pl = _pool(Q, fmt, w_["N"], w_["K"], w_["group"], True, 7, POOL_BYTES)
            for M in M_list:
                xa = torch.from_numpy(S.activations(w_, M)).cuda().to(torch.bfloat16)
                act = "swiglu" if w_.get("swiglu") else None
                ms, _ = time_forward(Q, pl, xa, act, max(20, len(pl), args.steps // 4), 5, use_graph,
                                     warm_s=AUX_WARM_S, reps=3)
                b = alg_bytes(fmt, M, w_["N"], w_["K"], w_["group"], False, bool(act), w_.get("bias_std") is not None)
                fl = 2.0 * M * w_["N"] * w_["K"]
                others[f"{name}/M{M}"] = {"us": round(ms * 1e3, 2), "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                                          "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1)}
            del pl
            torch.cuda.empty_cache()
        # the other weight formats at the codebook prefill's shape (3072 x 3072, M = 2048),
        # default schedules, weights from a pool as above
        xp = torch.from_numpy(S.activations(wl5, 2048)).cuda().to(torch.bfloat16)
        for fmt, G, sym in (("int4", 128, True), ("int4", 128, False), ("mxfp4", 32, True), ("int8", 256, True)):
            pl = _pool(Q, fmt, wl5["N"], wl5["K"], G, sym, 8, POOL_BYTES)
            ms, _ = time_forward(Q, pl, xp, None, max(20, len(pl), args.steps // 4), 5, use_graph,
                                 warm_s=AUX_WARM_S, reps=3)
            fl = 2.0 * 2048 * wl5["N"] * wl5["K"]
            tf = fl / (ms * 1e-3) / 1e12
            others[f"{fmt}{'' if sym else '_asym'}_g{G}_3072/M2048"] = {
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
    rec = {
        "metric": "W4A16 linear: effective HBM GB/s at M=1-16; TFLOP/s + MFMA util at M=2048",
        "value": round(value, 1),
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
                               "X bf16 [16,4096], bf16 out", "M": 16, "N": N, "K": K, "group": G,
                   "weight_pool_copies": n_copies, "hip_graph": use_graph, "schedule": repr(sched)},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "kernel": "qgemv_kernel (INT4, zero-points, group 128)", "alg_bytes": b16,
                     "us_per_launch": round(main_ms * 1e3, 3)},
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    if sweep:
        rec["sweep"] = sweep
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
