#!/usr/bin/env python3
"""Benchmark of the decode hot path on one MI355X: activation quantization + Q4_K GEMV.

One step = the whole hot path on one batch of synthetic input, through qgemv_fused: the
float32 activation is quantized to int8 blocks of 32 with float32 scales (written out as well)
and the block-quantized GEMV y = W x is computed from them. The library runs this as one
launch (each workgroup quantizing the columns it reads) or, when the activation slice is large
next to a workgroup's share of the weights, as qgemv_quantize_act then the product. The
explicit two-launch form and the GEMV alone are timed beside it. The default workload is the vocabulary projection, Q4_K W 262144 x 1536, batch 1:
weights N(0, 0.02) with 1% of the rows scaled by 10, quantized once by the library's
load-time quantizer; x N(0, 1).

Cold weights: the weight tensor is copied until the copies total >= 640 MB and the steps
rotate through them, so the 256 MB memory-side cache cannot hold the weights between uses
and the reads come from HBM. Inputs are resident in HBM before the timed region.

Prints ONE JSON line (rank 0, N = 1):
  value         whole-step algorithmic bytes / step time, GB/s
  roofline      the step's dominant kernel (the fused kernel when the step is one launch, else
                its GEMV launch): algorithmic bytes per launch / its average launch duration
                (HIP events on the launch stream over a run of back-to-back launches),
                against 8000 GB/s; traffic from the committed rocprofv3 counter summary when
                it was taken on the current kernel source, else null
  cpu_baseline  the CPU oracle's integer GEMV on a bounded row sample of the same workload
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import itertools
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # dense fp16 matrix peak of MI355X
MFMA_I8_PEAK_TOPS = 5000.0        # dense int8 matrix peak of MI355X (POP/s)
FORMAT_NAMES = {"q4k": "Q4_K", "q6k": "Q6_K", "q40": "Q4_0", "q80": "Q8_0"}
CALIB_COPY_BYTES = 256 << 20
COLD_BYTES = 640 * 10**6
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --traffic-calibration' into profiles/gemv_<workload>_traffic.json")
    ap.add_argument("--summarize-trace", nargs="+", metavar="CSV",
                    help="print a markdown table of a rocprofv3 --kernel-trace --stats summary "
                         "(KERNEL_STATS_CSV); with the run's KERNEL_TRACE_CSV as well, also the "
                         "average of each kernel over its dispatches after the warmup")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="q4k_262144x1536")
    ap.add_argument("--nvec", type=int, default=0,
                    help="override the workload's vector count (more than 8: matrix cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--warm", action="store_true", help="reuse one weight copy (cache-warm)")
    ap.add_argument("--counters", action="store_true",
                    help="for hardware-counter runs: skip the graph-replay phases (their "
                         "launches are the direct ones again) so each counter pass profiles "
                         "fewer dispatches")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="also run the read probe over one weight copy and a plain 256 MiB "
                         "device copy, the known-size kernels the HBM counters are scaled by")
    return ap.parse_args()


def kernel_sources(unit: str) -> list:
    """The source files of one kernel translation unit in csrc/: the unit and every file it
    includes from csrc/ (recursively), sorted."""
    csrc = os.path.join(ROOT, "block_quantized_weight_act_amd", "csrc")
    seen, todo = set(), [unit]
    while todo:
        name = todo.pop()
        if name in seen or not os.path.exists(os.path.join(csrc, name)):
            continue
        seen.add(name)
        with open(os.path.join(csrc, name)) as f:
            todo += re.findall(r'^#include "([^"]+)"', f.read(), flags=re.M)
    return sorted(seen)


def kernel_source_hash(unit: str = "gemv_q4k.hip") -> str:
    """SHA-256 over the sources the kernel is compiled from (default: the Q4_K GEMV kernels),
    so counters taken on those kernels stay valid while other files change."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_weight_act_amd", "csrc")
    for name in kernel_sources(unit):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def kernel_unit(kname: str) -> str:
    """The translation unit in csrc/ a kernel (as named in traces) is compiled from."""
    if kname.startswith("gemm_q4k_i8_kernel"):
        return "gemm_i8.hip"
    if kname.startswith("gemm_q4k_mfma_kernel") or kname.startswith("mc_stage_kernel"):
        return "gemm_mfma.hip"
    if kname.startswith("gemm_q32_mc_kernel"):
        return "gemm_q32.hip"
    if kname.startswith("gemm_q32_i8_kernel"):
        return "gemm_q32_i8.hip"
    if kname.startswith("gemm_q6k_mc_kernel"):
        return "gemm_q6k_mc.hip"
    for tag, unit in (("Q4K", "gemv_q4k.hip"), ("Q6K", "gemv_q6k.hip"), ("Q40", "gemv_q40.hip"),
                      ("Q80", "gemv_q80.hip")):
        if "qgemv::%s," % tag in kname:
            return unit
    raise ValueError("no translation unit known for kernel %r" % kname)


def load_traffic(workload: str, kname: str):
    """HBM bytes per launch of kernel `kname` from the committed rocprofv3 counter summary of
    the workload, or None when the summary is missing, covers another kernel, or was taken on
    other sources of that kernel."""
    path = os.path.join(PROFILES, "gemv_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kname:
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(kernel_unit(kname)):
        return None
    return rec.get("hbm_bytes_per_launch")


def weight_copies(w0, wbytes: int, warm: bool):
    """The rotating weight copies: (list of copies, count, keep-alive). Enough copies to total
    at least COLD_BYTES, so the 256 MB memory-side cache cannot hold the weights between uses.
    Up to 128 copies are separate tensors; more (small matrices) are 256-byte aligned slots of
    one buffer, passed as device pointers."""
    import torch
    if warm:
        return [w0], 1, None
    copies = max(1, math.ceil(COLD_BYTES / wbytes))
    if copies <= 128:
        return [w0] + [w0.clone() for _ in range(copies - 1)], copies, None
    stride = (wbytes + 255) // 256 * 256
    big = torch.empty(copies * stride, dtype=torch.uint8, device=w0.device)
    big[:wbytes].copy_(w0)
    filled = 1
    while filled < copies:
        n = min(filled, copies - filled)
        big[filled * stride:(filled + n) * stride].copy_(big[:n * stride])
        filled += n
    base = big.data_ptr()
    return [base + k * stride for k in range(copies)], copies, big


class Marks:
    """One-workgroup 16-byte read probes that cut the kernel trace into named windows, so a
    trace summary can average each kernel over exactly the dispatches of one measured phase."""

    def __init__(self, qg, dev):
        import torch
        self.qg = qg
        self.buf = torch.zeros(16, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)
        self.names = []

    def mark(self, name_of_next_window: str):
        self.qg.qgemv_read_probe(self.buf, self.sink, blocks=1, nbytes=16)
        self.names.append(name_of_next_window)


def algorithmic_bytes(wl, wbytes: int) -> dict:
    """Bytes each piece must move at least once. GEMV: the weights, the activation codes and
    scales, y. Quantization: the float32 activation in, codes and scales out. Step (the whole
    path): the weights and the float32 activation in, codes, scales and y out."""
    codes = wl.nvec * wl.cols + wl.nvec * (wl.cols // 32) * 4
    gemv = wbytes + codes + wl.nvec * wl.rows * 4
    quant = wl.nvec * wl.cols * 4 + codes
    step = wbytes + wl.nvec * wl.cols * 4 + codes + wl.nvec * wl.rows * 4
    return {"gemv": gemv, "quantize_act": quant, "step": step}


def roofline_kernel(wtype: str, plan: dict, nvec: int, launches: int, route: str = "vector") -> str:
    """The step's dominant kernel, as its template instance appears in kernel traces: the
    one-launch fused kernel (form 2) when qgemv_fused makes one launch for this shape, else the
    GEMV kernel of the two-launch route (form 0, codes read from memory; for a plan with
    column splits the kernel that splits inside the workgroup); on the integer matrix-core
    route the product kernel of that route."""
    if route == "i8mc":
        # the third template argument (operands kept in registers or not) is chosen at launch
        # from the GPU's occupancy, so the name is given up to it (a prefix of the trace name)
        return "gemm_q4k_i8_kernel<%d, %d, " % (2 if launches == 1 else 0, (nvec + 7) // 8)
    if route == "mc32" and nvec <= 8:
        # the few-vector integer matrix-core kernel (format, form from codes, halves of 4
        # vectors; the last argument, one scale load per lane, follows the row width)
        return "gemm_q32_i8_kernel<%d, 0, %d, " % ({"q6k": 2, "q40": 3, "q80": 4}[wtype],
                                                   (nvec + 3) // 4)
    tag = {"q4k": "Q4K", "q6k": "Q6K", "q40": "Q40", "q80": "Q80"}[wtype]
    if launches != 1 and plan["splits"] > 1:
        # the unfused product of a split plan: the column split inside the workgroup
        return "gemv_split_kernel<qgemv::%s, %d, %d, %d>" % (tag, nvec, plan["lanes_per_row"],
                                                           plan["chunks_per_lane"])
    return "gemv_kernel<qgemv::%s, %d, %d, %d, %d>" % (tag, nvec, plan["lanes_per_row"],
                                                       plan["chunks_per_lane"],
                                                       2 if launches == 1 else 0)


def cpu_baseline(wl, seconds: float, y_gpu: np.ndarray, max_rows: int = 32768) -> dict:
    """The oracle's GEMV timed on a bounded sample of rows; on the way it also checks the
    GPU's y on those rows against the oracle's error bound (untimed)."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    rows = min(wl.rows, max_rows)
    sample = np.linspace(0, wl.rows - 1, rows).astype(np.int64)
    w = wl.weight_rows(sample)
    wbuf = oracle.quantize(wl.wtype, w)
    xq, xd = oracle.quantize_act(wl.activations())
    ref = oracle.gemv(wl.wtype, wbuf, rows, wl.cols, xq, xd)
    err = np.abs(y_gpu[:, sample].astype(np.float64) - ref["y"])
    ratio = float(np.max(err / np.maximum(ref["bound"], np.finfo(np.float64).tiny)))
    nbytes = wbuf.size + xq.size + xd.size * 4 + wl.nvec * rows * 4

    def rate(nthreads, budget):
        oracle.gemv_threaded(wl.wtype, wbuf, rows, wl.cols, xq, xd, nthreads)   # warm-up
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.gemv_threaded(wl.wtype, wbuf, rows, wl.cols, xq, xd, nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return el / reps, reps, el

    per, reps, el = rate(threads, seconds)
    per1, reps1, el1 = rate(1, seconds / 2)
    # the oracle's activation quantizer on the workload's activation, timed on its own (one
    # thread; it is a few microseconds per call, so many calls are timed together)
    x_act = wl.activations()
    oracle.quantize_act(x_act)
    qreps, q0 = 0, time.perf_counter()
    while True:
        for _ in range(100):
            oracle.quantize_act(x_act)
        qreps += 100
        qel = time.perf_counter() - q0
        if qel >= min(2.0, seconds / 4):
            break
    q_per = qel / qreps
    q_bytes = x_act.size * 4 + x_act.size + (x_act.size // 32) * 4
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d rows (evenly spaced), full width, %d reps in %.1f s on %d threads; "
                      "integer GEMV only, weights quantized beforehand" % (rows, wl.rows, reps, el,
                                                                          threads),
            "us_per_gemv_scaled_to_full": round(per * (wl.rows / rows) * 1e6, 1),
            "one_core": {"value": round(nbytes / per1 / 1e9, 3), "unit": "GB/s", "reps": reps1,
                         "seconds": round(el1, 1)},
            "cpu_model": model,
            "quantize_act": {"us_per_call": round(q_per * 1e6, 3),
                             "gbs": round(q_bytes / q_per / 1e9, 3), "cores": 1,
                             "calls": qreps, "seconds": round(qel, 2),
                             "sample": "the workload's whole activation (%d vectors x %d "
                                       "columns) per call, including the Python binding's "
                                       "copies" % (wl.nvec, wl.cols)},
            "gpu_y_check": {"rows": rows, "max_err_over_bound": ratio, "ok": ratio <= 1.0}}


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_traffic(args) -> None:
    """HBM bytes per GEMV launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for kernels of known size in the same run: the read probe over
    one weight copy (FETCH_SIZE) and the last ten plain 256 MiB device copies (WRITE_SIZE)."""
    import synth
    wl = synth.WORKLOADS[args.workload]
    import block_quantized_weight_act_amd as qg
    wbytes = qg.qgemv_weight_bytes(wl.wtype, wl.rows, wl.cols)
    if wl.nvec > 8:
        # the product from codes (bench_many's roofline kernel): weights, codes and y
        launches = 2
        kname = many_kernel(qg, wl)
    else:
        launches = qg.qgemv_fused_launches(wl.wtype, wl.rows, wl.cols, wl.nvec, True)
        kname = roofline_kernel(wl.wtype, qg.qgemv_plan_for(wl.wtype, wl.rows, wl.cols, wl.nvec),
                                wl.nvec, launches, qg.qgemv_route(wl.wtype, wl.rows, wl.cols, wl.nvec))
    per = {}
    for path, counter in zip(args.summarize_traffic, ("FETCH_SIZE", "WRITE_SIZE")):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == counter]
        gemv = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]]
        # read probes over one whole weight copy (not the one-workgroup warmup marker)
        probe = [float(r["Counter_Value"]) for r in rows if "read_probe_kernel" in r["Kernel_Name"]
                 and int(r["Grid_Size"]) > int(r["Workgroup_Size"])]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-10:]
        per[counter] = {"gemv_kib": sum(gemv) / len(gemv), "gemv_dispatches": len(gemv),
                        "probe_kib": sum(probe) / len(probe), "copy_kib": sum(copies) / len(copies)}
    f = per["FETCH_SIZE"]
    w = per["WRITE_SIZE"]
    fetch_factor = wbytes / (f["probe_kib"] * 1024)
    fetch_factor_copy = CALIB_COPY_BYTES / (f["copy_kib"] * 1024)
    write_factor = CALIB_COPY_BYTES / (w["copy_kib"] * 1024)
    hbm = f["gemv_kib"] * 1024 * fetch_factor + w["gemv_kib"] * 1024 * write_factor
    alg = algorithmic_bytes(wl, wbytes)["step" if launches == 1 else "gemv"]
    rec = {
        "workload": wl.name, "kernel": kname,
        "kernel_source_sha256": kernel_source_hash(kernel_unit(kname)),
        "fetch_size_kib_per_dispatch": round(f["gemv_kib"], 3),
        "write_size_kib_per_dispatch": round(w["gemv_kib"], 3),
        "fetch_factor": round(fetch_factor, 6),
        "fetch_factor_from_copy": round(fetch_factor_copy, 6),
        "write_factor": round(write_factor, 6),
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": alg,
        "ratio_to_algorithmic": round(hbm / alg, 5),
        "dispatches": f["gemv_dispatches"],
    }
    path = os.path.join(PROFILES, "gemv_%s_traffic.json" % wl.name)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def summarize_trace(paths: list) -> None:
    """rocprofv3's per-kernel summary, then per-dispatch averages in each measured window. The
    bench cuts the trace into windows with one-workgroup read probes (Marks); the warmup before
    the first mark is left out. A third path, a file holding the bench's JSON line, names the
    windows (its trace_windows)."""
    rows = _counter_rows(paths[0])
    print("| kernel | calls | average us | min us | max us | stddev us | % of GPU time |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        print("| `%s` | %s | %.3f | %.3f | %.3f | %.3f | %s |" % (
            r["Name"], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["StdDev"]) / 1e3, r["Percentage"]))
    if len(paths) < 2:
        return
    names = []
    if len(paths) > 2:
        with open(paths[2]) as f:
            line = next(ln for ln in f if ln.lstrip().startswith("{"))
        names = json.loads(line).get("trace_windows", [])
    trace = sorted(_counter_rows(paths[1]), key=lambda r: int(r["Start_Timestamp"]))
    windows, cur = [], None
    for r in trace:
        if "read_probe_kernel" in r["Kernel_Name"] and r["Grid_Size_X"] == r["Workgroup_Size_X"]:
            cur = {}
            windows.append(cur)
            continue
        if cur is None:
            continue                              # the warmup
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        cur.setdefault(r["Kernel_Name"], []).append(d)
    print()
    print("| window (between the bench's marks) | kernel | dispatches | average us | median us |")
    print("|---|---|---|---|---|")
    for k, per in enumerate(windows):
        label = names[k] if k < len(names) else "window %d" % (k + 1)
        for name, ds in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            ds = sorted(ds)
            print("| %s | `%s` | %d | %.3f | %.3f |" % (label, name, len(ds), sum(ds) / len(ds),
                                                       ds[len(ds) // 2]))


def timed(fn, n):
    """ms per launch (HIP events on the current stream) and host wall ms per launch of n
    back-to-back launches, after 50 of the same."""
    import torch
    for i in range(min(n, 50)):           # this form's own short warmup
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    w0_ = time.perf_counter()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0_
    return e0.elapsed_time(e1) / n, wall / n * 1e3

def spread(fn, n, batches=20):
    """Per-launch time in each of `batches` consecutive batches of back-to-back launches
    (one event pair per batch, so no per-launch event overhead): p10, median, p90 (us)."""
    import torch
    per = max(1, n // batches)
    for i in range(min(n, 50)):
        fn(i)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for b in range(batches):
        for i in range(per):
            fn(b * per + i)
        evs[b + 1].record()
    torch.cuda.synchronize()
    d = sorted(evs[b].elapsed_time(evs[b + 1]) * 1e3 / per for b in range(batches))
    return {"batches": batches, "launches_per_batch": per, "p10": round(d[batches // 10], 3),
            "median": round(d[batches // 2], 3), "p90": round(d[(9 * batches) // 10], 3)}

def capture(fn, n):
    """The same launches captured once into a HIP graph (replayed, they give the GPU time
    per launch without the host's per-call overhead, as a decode loop replaying a graph
    sees it)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g

def replay_timed(g, n):
    import torch
    g.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def bench_group(args) -> dict:
    """Several matrices sharing one activation (a multi-matrix workload). Step = one launch of
    qgemv_multi_fused (the float32 activation quantized inside, every matrix's y out). Beside
    it: the same product from codes (qgemv_multi), one qgemv_fused per matrix, and
    quantize-then-one-GEMV-per-matrix."""
    import torch

    import block_quantized_weight_act_amd as qg
    import synth

    grp = synth.GROUPS[args.workload]
    cols, nvec = grp.cols, grp.nvec
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    tensors = []
    for p in grp.parts:
        wb = qg.qgemv_weight_bytes(p.wtype, p.rows, cols)
        w0 = torch.empty(wb, dtype=torch.uint8, device=dev)
        for r0 in range(0, p.rows, 32768):
            r1 = min(p.rows, r0 + 32768)
            wf = torch.from_numpy(p.weight_block(r0, r1)).to(dev)
            qg.qgemv_quantize_weights_rows(p.wtype, wf, w0, p.rows, cols, r0, r1 - r0)
            del wf
        tensors.append(w0)
    wbytes = sum(t.numel() for t in tensors)
    copies = 1 if args.warm else max(1, min(256, math.ceil(COLD_BYTES / wbytes)))
    sets = [tensors] + [[t.clone() for t in tensors] for _ in range(copies - 1)]
    x = torch.from_numpy(grp.activations()).to(dev)
    xq = torch.empty((nvec, cols), dtype=torch.int8, device=dev)
    xd = torch.empty((nvec, cols // 32), dtype=torch.float32, device=dev)
    ys = [torch.empty((nvec, p.rows), dtype=torch.float32, device=dev) for p in grp.parts]
    work = [torch.empty(max(4, qg.qgemv_workspace_bytes(p.wtype, p.rows, cols, nvec)),
                        dtype=torch.uint8, device=dev) for p in grp.parts]
    mats = [[(p.wtype, st[k], p.rows, ys[k]) for k, p in enumerate(grp.parts)] for st in sets]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def step(i):
        qg.qgemv_multi_fused(mats[i % copies], x, cols, nvec)

    def multi(i):
        qg.qgemv_multi(mats[i % copies], xq, xd, cols, nvec)

    def fused_each(i):
        for k, p in enumerate(grp.parts):
            qg.qgemv_fused(p.wtype, sets[i % copies][k], x, ys[k], p.rows, cols, nvec,
                           workspace=work[k])

    def separate(i):
        qg.qgemv_quantize_act(x, xq, xd, cols, nvec)
        for k, p in enumerate(grp.parts):
            qg.qgemv_batch(p.wtype, sets[i % copies][k], xq, xd, ys[k], p.rows, cols, nvec,
                           workspace=work[k])

    forms = (("step", step), ("multi", multi), ("fused_each", fused_each), ("separate", separate))
    graphs = {name: capture(fn, args.steps) for name, fn in forms}
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sink_mark = torch.zeros(16, dtype=torch.uint8, device=dev)
    for _ in range(2):
        for st in sets:
            for t in st:
                qg.qgemv_read_probe(t, sink, blocks=4096)
    separate(0)            # makes the codes the multi form reads
    for i in range(args.warmup):
        step(i)
    qg.qgemv_read_probe(sink_mark, sink, blocks=1, nbytes=16)
    ms = {name: timed(fn, args.steps)[0] for name, fn in forms}
    ms_graph = {name: replay_timed(graphs[name], args.steps) for name, _ in forms}
    step_dist = spread(step, args.steps)
    step(0)
    torch.cuda.synchronize()
    if not all(bool(torch.isfinite(y).all()) for y in ys):
        print("bench.py: the product gave non-finite outputs", file=sys.stderr)
        sys.exit(1)

    codes = nvec * cols + nvec * (cols // 32) * 4
    ybytes = sum(nvec * p.rows * 4 for p in grp.parts)
    step_bytes = wbytes + nvec * cols * 4 + ybytes
    multi_bytes = wbytes + codes + ybytes
    t, nc = qg.qgemv_multi_geometry(cols, nvec)
    achieved = step_bytes / (ms["step"] * 1e-3) / 1e9
    roof_gbs = step_bytes / (ms_graph["step"] * 1e-3) / 1e9
    # one format: the one-format walk; several: the kernel that splits its grid between them
    formats = sorted({p.wtype for p in grp.parts})
    if len(formats) == 1:
        multi_kernel = "gemv_multi_fmt_kernel<qgemv::%s, %d, %d, %d, 2>" % (
            {"q4k": "Q4K", "q6k": "Q6K", "q40": "Q40", "q80": "Q80"}[formats[0]], nvec, t, nc)
    else:
        multi_kernel = "gemv_multi_kernel<%d, %d, %d, 2>" % (nvec, t, nc)
    out = {
        "metric": "achieved HBM GB/s and % of roofline, multi-matrix GEMV sharing one activation",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms["step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xq4k/q6k",
        "data": "synthetic",
        "config": {"workload": "%d matrices sharing one activation, %s, cols %d, batch %d, cold "
                               "weights (%d rotating copies)" % (
                                   len(grp.parts), " + ".join("%s %d" % (FORMAT_NAMES[p.wtype], p.rows)
                                                              for p in grp.parts),
                                   cols, nvec, copies),
                   "name": grp.name, "cols": cols, "nvec": nvec, "weight_bytes": wbytes,
                   "lanes_per_row": t, "chunks_per_lane": nc},
        "us_per_step": round(ms["step"] * 1e3, 3),
        "us_per_multi_from_codes": round(ms["multi"] * 1e3, 3),
        "us_per_fused_each": round(ms["fused_each"] * 1e3, 3),
        "us_per_separate": round(ms["separate"] * 1e3, 3),
        "graph_replay": {"us_per_step": round(ms_graph["step"] * 1e3, 3),
                         "us_per_multi_from_codes": round(ms_graph["multi"] * 1e3, 3),
                         "us_per_fused_each": round(ms_graph["fused_each"] * 1e3, 3),
                         "us_per_separate": round(ms_graph["separate"] * 1e3, 3)},
        "us_per_step_distribution": step_dist,
        "roofline": {"bound": "hbm", "achieved": round(roof_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(roof_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": multi_kernel,
                     "algorithmic_bytes_per_launch": step_bytes,
                     "us_per_launch": round(ms_graph["step"] * 1e3, 3),
                     "statistic": "mean launch time over a graph replay of back-to-back steps "
                                  "(HIP events on the replay stream)"},
        "multi_from_codes_gbs": round(multi_bytes / (ms["multi"] * 1e-3) / 1e9, 1),
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_group(grp, args.cpu_seconds,
                                                 [y.cpu().numpy() for y in ys])
    return out


def cpu_baseline_group(grp, seconds: float, y_gpu: list) -> dict:
    """The oracle's GEMV over every matrix of the group (all rows), timed; on the way each
    GPU y is checked against the oracle's error bound (untimed)."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    xq, xd = oracle.quantize_act(grp.activations())
    bufs, ratio = [], 0.0
    for p, yg in zip(grp.parts, y_gpu):
        w = p.weight_block(0, p.rows)
        buf = oracle.quantize(p.wtype, w)
        ref = oracle.gemv(p.wtype, buf, p.rows, grp.cols, xq, xd)
        err = np.abs(yg.astype(np.float64) - ref["y"])
        ratio = max(ratio, float(np.max(err / np.maximum(ref["bound"], np.finfo(np.float64).tiny))))
        bufs.append(buf)
    nbytes = sum(b.size for b in bufs) + xq.size + xd.size * 4 + sum(grp.nvec * p.rows * 4
                                                                    for p in grp.parts)

    def once():
        for p, b in zip(grp.parts, bufs):
            oracle.gemv_threaded(p.wtype, b, p.rows, grp.cols, xq, xd, threads)

    once()
    reps, t0 = 0, time.perf_counter()
    while True:
        once()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(nbytes / (el / reps) / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": "every row of every matrix, %d reps in %.1f s on %d "
                                        "threads" % (reps, el, threads),
            "gpu_y_check": {"max_err_over_bound": ratio, "ok": ratio <= 1.0}}


def bench_decode(args) -> dict:
    """A whole decode step's products (every layer, then the vocabulary projection), recorded
    once with qgemv_graph_begin / qgemv_graph_end and replayed with one qgemv_graph_launch per
    step. Step = one replay. Beside it: the same calls made directly from Python, and a
    per-matrix form (quantize, then one product per matrix) replayed as a graph too."""
    import torch

    import block_quantized_weight_act_amd as qg
    import synth

    dec = synth.DECODE_STEPS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    items, wbytes, ws_bytes, codes_bytes, y_bytes, x_bytes = [], 0, 16, 0, 0, 0
    for kind, item in dec.products():
        parts = item.parts if kind == "multi" else (item,)
        cols, nvec = parts[0].cols, parts[0].nvec
        ws = []
        for p in parts:
            w0 = torch.empty(qg.qgemv_weight_bytes(p.wtype, p.rows, cols), dtype=torch.uint8,
                             device=dev)
            for r0 in range(0, p.rows, 32768):
                r1 = min(p.rows, r0 + 32768)
                wf = torch.from_numpy(p.weight_block(r0, r1)).to(dev)
                qg.qgemv_quantize_weights_rows(p.wtype, wf, w0, p.rows, cols, r0, r1 - r0)
                del wf
            ws.append(w0)
            wbytes += w0.numel()
            ws_bytes = max(ws_bytes, qg.qgemv_workspace_bytes(p.wtype, p.rows, cols, nvec))
        x = torch.from_numpy(parts[0].activations()).to(dev)
        x_bytes += x.numel() * 4
        codes_bytes += nvec * cols + nvec * (cols // 32) * 4
        ys = [torch.empty((nvec, p.rows), dtype=torch.float32, device=dev) for p in parts]
        y_bytes += sum(y.numel() * 4 for y in ys)
        xq = torch.empty((nvec, cols), dtype=torch.int8, device=dev)
        xd = torch.empty((nvec, cols // 32), dtype=torch.float32, device=dev)
        items.append((kind, parts, ws, x, ys, xq, xd))
    work = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def step():
        for kind, parts, ws, x, ys, xq, xd in items:
            cols, nvec = parts[0].cols, parts[0].nvec
            if kind == "multi":
                qg.qgemv_multi_fused([(p.wtype, w, p.rows, y) for p, w, y in zip(parts, ws, ys)],
                                     x, cols, nvec)
            else:
                p = parts[0]
                qg.qgemv_fused(p.wtype, ws[0], x, ys[0], p.rows, cols, nvec, workspace=work)

    def per_matrix():
        for kind, parts, ws, x, ys, xq, xd in items:
            cols, nvec = parts[0].cols, parts[0].nvec
            qg.qgemv_quantize_act(x, xq, xd, cols, nvec)
            for p, w, y in zip(parts, ws, ys):
                qg.qgemv_batch(p.wtype, w, xq, xd, y, p.rows, cols, nvec, workspace=work)

    def record(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()                                  # once directly on the capture stream
            qg.qgemv_graph_begin()
            fn()
            g = qg.qgemv_graph_end()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    g_step, g_per = record(step), record(per_matrix)
    launches, others = g_step.nodes()
    launches_per, _ = g_per.nodes()
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sink_mark = torch.zeros(16, dtype=torch.uint8, device=dev)
    for kind, parts, ws, *_ in items:
        for w in ws:
            qg.qgemv_read_probe(w, sink, blocks=1024)
    for _ in range(args.warmup):
        g_step.launch()
    qg.qgemv_read_probe(sink_mark, sink, blocks=1, nbytes=16)

    def events(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w = time.perf_counter()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, (time.perf_counter() - w) * 1e3 / n

    ms_step, wall_step = events(g_step.launch, args.steps)
    dist = spread(lambda i: g_step.launch(), args.steps)
    for _ in range(20):
        g_per.launch()
    ms_per, _ = events(g_per.launch, max(20, args.steps // 4))
    for _ in range(5):
        step()
    ms_direct, wall_direct = events(step, max(10, args.steps // 10))
    g_step.launch()
    torch.cuda.synchronize()
    ys_all = [y for it in items for y in it[4]]
    if not all(bool(torch.isfinite(y).all()) for y in ys_all):
        print("bench.py: the decode step gave non-finite outputs", file=sys.stderr)
        sys.exit(1)
    step_bytes = wbytes + x_bytes + y_bytes
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    nl = len(dec.layers)
    out = {
        "metric": "achieved HBM GB/s and % of roofline, whole decode step of GEMVs replayed as one "
                  "graph",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xq4k/q6k",
        "data": "synthetic",
        "config": {"workload": "decode step: %d layers x (QKV %d/%d/%d, O %dx%d, gate+up 2x%dx%d, "
                               "down %dx%d) + head %dx%d, batch 1" % (
                                   nl, *[p.rows for p in dec.layers[0].qkv.parts],
                                   dec.layers[0].o.rows, dec.layers[0].o.cols,
                                   dec.layers[0].gate_up.parts[0].rows, dec.layers[0].gate_up.cols,
                                   dec.layers[0].down.rows, dec.layers[0].down.cols,
                                   dec.head.rows, dec.head.cols),
                   "name": dec.name, "layers": nl, "weight_bytes": wbytes,
                   "graph_kernel_launches": launches, "graph_other_nodes": others},
        "us_per_step": round(ms_step * 1e3, 3),
        "tokens_per_s_gemv_only": round(1e3 / ms_step, 1),
        "us_per_step_distribution": dist,
        "host_us_per_graph_launch": round(wall_step * 1e3, 3),
        "direct_calls": {"us_per_step": round(ms_direct * 1e3, 3),
                         "host_us_per_step": round(wall_direct * 1e3, 3),
                         "calls_per_step": len(items)},
        "per_matrix_graph": {"us_per_step": round(ms_per * 1e3, 3),
                             "kernel_launches": launches_per,
                             "gbs": round((wbytes + x_bytes + y_bytes + 2 * codes_bytes)
                                          / (ms_per * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode-step graph (%d kernel launches)" % launches,
                     "algorithmic_bytes_per_launch": step_bytes,
                     "us_per_launch": round(ms_step * 1e3, 3)},
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        l0 = dec.layers[0]
        grp_like = [(l0.qkv.parts, items[0]), ((l0.o,), items[1]), (l0.gate_up.parts, items[2]),
                    ((l0.down,), items[3])]
        out["cpu_baseline"] = cpu_baseline_decode_layer(grp_like, args.cpu_seconds)
    g_step.close()
    g_per.close()
    return out


def cpu_baseline_decode_layer(products, seconds: float) -> dict:
    """The oracle over layer 0's seven matrices (every row, each on its own activation),
    timed; on the way the GPU's y of those products is checked against the oracle's error bound
    (untimed)."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    work, ratio, nbytes = [], 0.0, 0
    for parts, (kind, _, _, x, ys, _, _) in products:
        cols = parts[0].cols
        xq, xd = oracle.quantize_act(parts[0].activations())
        nbytes += xq.size + xd.size * 4
        for p, yg in zip(parts, ys):
            buf = oracle.quantize(p.wtype, p.weight_block(0, p.rows))
            ref = oracle.gemv(p.wtype, buf, p.rows, cols, xq, xd)
            err = np.abs(yg.cpu().numpy().astype(np.float64) - ref["y"])
            ratio = max(ratio, float(np.max(err / np.maximum(ref["bound"],
                                                              np.finfo(np.float64).tiny))))
            work.append((p.wtype, buf, p.rows, cols, xq, xd))
            nbytes += buf.size + p.nvec * p.rows * 4

    def once():
        for wtype, buf, rows, cols, xq, xd in work:
            oracle.gemv_threaded(wtype, buf, rows, cols, xq, xd, threads)

    once()
    reps, t0 = 0, time.perf_counter()
    while True:
        once()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(nbytes / (el / reps) / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": "layer 0's seven matrices, every row, %d reps in %.1f s "
                                        "on %d threads" % (reps, el, threads),
            "gpu_y_check": {"max_err_over_bound": ratio, "ok": ratio <= 1.0}}


def many_kernel(qg, wl) -> str:
    """The product kernel of a workload with more than 8 vectors, as its template instance
    appears in kernel traces (a prefix where an argument is chosen at launch)."""
    rows, cols, nvec = wl.rows, wl.cols, wl.nvec
    route = qg.qgemv_route(wl.wtype, rows, cols, nvec)
    if route == "i8mc":
        # the integer matrix cores (int8 products; 9..16 vectors)
        return "gemm_q4k_i8_kernel<0, %d, " % ((nvec + 7) // 8)
    if route == "mc32" and qg.qgemv_mc32_tile(wl.wtype, rows, cols, nvec) == 16:
        # the 16 x 16 x 64 kernel (format, form from codes, halves of 4 vectors; the last
        # argument follows the row width)
        return "gemm_q32_i8_kernel<%d, 0, %d, " % ({"q4k": 1, "q6k": 2, "q40": 3, "q80": 4}[wl.wtype],
                                                    (nvec + 3) // 4)
    if route == "mc32":
        # the workgroup shape by vector tiles (1, 2, 4): Q8_0 / Q4_0 rows, vector groups, tiles
        # per wave; Q6_K row groups, vector tiles, row tiles per wave; then blocks per step
        vtiles = (nvec + 31) // 32
        vt = 4 if vtiles >= 3 else vtiles
        if wl.wtype == "q6k":
            return "gemm_q6k_mc_kernel<%d, %d, %d, 8, false>" % {1: (4, 1, 1), 2: (2, 2, 2),
                                                                  4: (1, 4, 2)}[vt]
        ks = 4 if wl.wtype == "q40" and vt == 2 else 8
        return "gemm_q32_mc_kernel<%d, %d, %d, %d, %d, false>" % (
            (4 if wl.wtype == "q80" else 3,) + {1: (4, 1, 1), 2: (4, 1, 2), 4: (2, 2, 2)}[vt] + (ks,))
    # the library's tile rule: one group of ceil(nvec / 32) tiles up to 96 vectors, else 2
    return "gemm_q4k_mfma_kernel<%d, false>" % ((nvec + 31) // 32 if nvec <= 96 else 2)


def bench_many(args, wl) -> dict:
    """More than 8 vectors (the matrix-core kernel). Step = qgemv_quantize_act + qgemv_batch
    (plus the ordered reduce when the super-blocks are split), replayed as one graph over
    rotating weight copies. Beside it: the product alone, and the same vectors in groups of 8
    (ceil(nvec / 8) products, each reading all the weights) through the vector kernel and
    through the integer matrix-core kernel."""
    import torch

    import block_quantized_weight_act_amd as qg

    nvec, rows, cols = wl.nvec, wl.rows, wl.cols
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    wbytes = qg.qgemv_weight_bytes(wl.wtype, rows, cols)
    w0 = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    for r0 in range(0, rows, 32768):
        r1 = min(rows, r0 + 32768)
        wf = torch.from_numpy(wl.weight_block(r0, r1)).to(dev)
        qg.qgemv_quantize_weights_rows(wl.wtype, wf, w0, rows, cols, r0, r1 - r0)
        del wf
    copies = 1 if args.warm else max(1, min(64, math.ceil(COLD_BYTES / wbytes)))
    ws_list = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(wl.activations()).to(dev)
    xq = torch.empty((nvec, cols), dtype=torch.int8, device=dev)
    xd = torch.empty((nvec, cols // 32), dtype=torch.float32, device=dev)
    y = torch.empty((nvec, rows), dtype=torch.float32, device=dev)
    wsb = max(qg.qgemv_workspace_bytes(wl.wtype, rows, cols, nvec),
              qg.qgemv_workspace_bytes(wl.wtype, rows, cols, 8))
    work = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def gemm(i):
        qg.qgemv_batch(wl.wtype, ws_list[i % copies], xq, xd, y, rows, cols, nvec, workspace=work)

    def step(i):
        qg.qgemv_quantize_act(x, xq, xd, cols, nvec)
        gemm(i)

    plans = {n: qg.qgemv_plan_for(wl.wtype, rows, cols, n) for n in range(1, 9)}
    wsb = max(wsb, max(qg.qgemv_plan_workspace_bytes(p, rows, cols, n) for n, p in plans.items()),
              qg.qgemv_i8mc_workspace_bytes(rows, cols, 8))
    work = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)

    def by_eight(i):
        # the vector kernel (its own plan) on groups of 8 vectors
        for v0 in range(0, nvec, 8):
            n = min(8, nvec - v0)
            qg.qgemv_batch_plan(wl.wtype, ws_list[i % copies], xq[v0:v0 + n], xd[v0:v0 + n],
                                y[v0:v0 + n], rows, cols, n, plans[n], workspace=work)

    def by_eight_i8(i):
        # the integer matrix-core kernel on groups of 8 vectors
        for v0 in range(0, nvec, 8):
            n = min(8, nvec - v0)
            qg.qgemv_batch_i8mc(ws_list[i % copies], xq[v0:v0 + n], xd[v0:v0 + n],
                                y[v0:v0 + n], rows, cols, n, workspace=work)

    n8 = max(4, args.steps // 8)
    graphs = {"step": capture(step, args.steps), "gemm": capture(gemm, args.steps),
              "by_eight": capture(by_eight, n8)}
    if wl.wtype == "q4k":                 # the integer matrix-core kernel of groups takes Q4_K
        graphs["by_eight_i8"] = capture(by_eight_i8, n8)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sink_mark = torch.zeros(16, dtype=torch.uint8, device=dev)
    for _ in range(2):
        for t in ws_list:
            qg.qgemv_read_probe(t, sink, blocks=4096)
    for i in range(args.warmup):
        step(i)
    qg.qgemv_read_probe(sink_mark, sink, blocks=1, nbytes=16)
    ms_step = replay_timed(graphs["step"], args.steps)
    ms_gemm = replay_timed(graphs["gemm"], args.steps)
    ms_gemm_events, _ = timed(gemm, args.steps)
    ms_eight = replay_timed(graphs["by_eight"], n8)
    ms_eight_i8 = replay_timed(graphs["by_eight_i8"], n8) if "by_eight_i8" in graphs else None
    dist = spread(step, args.steps)
    step(0)
    torch.cuda.synchronize()
    if not bool(torch.isfinite(y).all()):
        print("bench.py: the product gave non-finite outputs", file=sys.stderr)
        sys.exit(1)

    codes = nvec * cols + nvec * (cols // 32) * 4
    ybytes = nvec * rows * 4
    gemm_bytes = wbytes + codes + ybytes
    step_bytes = wbytes + nvec * cols * 4 + ybytes
    flops = 2.0 * rows * cols * nvec
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    gemm_gbs = gemm_bytes / (ms_gemm * 1e-3) / 1e9
    gemm_tflops = flops / (ms_gemm * 1e-3) / 1e12
    t_hbm = gemm_bytes / (HBM_PEAK_GBS * 1e9)
    route = qg.qgemv_route(wl.wtype, rows, cols, nvec)
    # The contraction is int8 codes x int8 (Q8_0), 6-bit (Q6_K) or 4-bit (Q4_K, Q4_0) codes, so every route
    # is set against the int8 matrix peak; the float route (fp16 products of exact integers)
    # is also given against its own fp16 peak.
    mfma_peak, mfma_unit = MFMA_I8_PEAK_TOPS, "TOP/s"
    kernel = many_kernel(qg, wl)
    t_mfma = flops / (mfma_peak * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(gemm_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": mfma_peak,
                "unit": mfma_unit, "frac": round(gemm_tflops / mfma_peak, 4)}
    roof.update({"traffic": None, "kernel": kernel, "algorithmic_bytes_per_launch": gemm_bytes,
                 "algorithmic_flops_per_launch": flops,
                 "us_per_launch": round(ms_gemm * 1e3, 3),
                 "hbm_frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(gemm_tflops / mfma_peak, 4), "route": route})
    if route == "mc":
        roof["mfma_f16_frac"] = round(gemm_tflops / MFMA_F16_PEAK_TFLOPS, 4)
    out = {
        "metric": "achieved HBM GB/s and % of roofline, block-quantized GEMV with many activation "
                  "vectors (matrix cores)",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8x" + wl.wtype,
        "data": "synthetic",
        "config": {"workload": "%s W %d x %d, %d vectors, cold weights (%d rotating copies)" % (
                       FORMAT_NAMES[wl.wtype], rows, cols, nvec, copies),
                   "name": wl.name, "rows": rows, "cols": cols, "nvec": nvec,
                   "weight_bytes": wbytes,
                   "workspace_bytes": qg.qgemv_workspace_bytes(wl.wtype, rows, cols, nvec)},
        "us_per_step": round(ms_step * 1e3, 3),
        "us_per_step_distribution": dist,
        "us_per_gemm": round(ms_gemm * 1e3, 3),
        "us_per_gemm_host_launched": round(ms_gemm_events * 1e3, 3),
        "gemm_gbs": round(gemm_gbs, 1),
        "gemm_tflops": round(gemm_tflops, 2),
        "roofline_floor_us": {"hbm": round(t_hbm * 1e6, 2), "mfma_i8": round(t_mfma * 1e6, 2)},
        "eight_vector_kernel": {"us_for_all_vectors": round(ms_eight * 1e3, 3),
                                "launches": (nvec + 7) // 8,
                                "speedup_of_matrix_cores": round(ms_eight / ms_gemm, 2)},
        "eight_vector_integer_matrix_cores": None if ms_eight_i8 is None else {
            "us_for_all_vectors": round(ms_eight_i8 * 1e3, 3), "launches": (nvec + 7) // 8,
            "speedup_of_matrix_cores": round(ms_eight_i8 / ms_gemm, 2)},
        "roofline": roof,
        "setup_s": round(setup_s, 1),
    }
    if args.traffic_calibration:
        # kernels of known size for the counters' scale (as in the main path): read probes
        # over one weight copy, then plain 256 MiB device copies
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for i in range(10):
            qg.qgemv_read_probe(ws_list[i % copies], sink, blocks=4096, nbytes=wbytes)
        src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["traffic_calibration"] = {"read_probe_bytes": wbytes, "copy_bytes": CALIB_COPY_BYTES}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, y.cpu().numpy(),
                                           max_rows=max(512, 32768 * 8 // nvec))
    return out


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import synth
    if args.workload in synth.GROUPS:
        print(json.dumps(bench_group(args)), flush=True)
        return
    if args.workload in synth.DECODE_STEPS:
        print(json.dumps(bench_decode(args)), flush=True)
        return
    import torch

    import block_quantized_weight_act_amd as qg

    wl = synth.WORKLOADS[args.workload]
    if args.nvec:
        wl = dataclasses.replace(wl, nvec=args.nvec, name="%s_n%d" % (wl.name, args.nvec))
    if wl.nvec > 8:
        print(json.dumps(bench_many(args, wl)), flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()

    # weights: generated on the host in row chunks, each quantized on the GPU into its place
    wbytes = qg.qgemv_weight_bytes(wl.wtype, wl.rows, wl.cols)
    w0 = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    chunk = 32768
    for r0 in range(0, wl.rows, chunk):
        r1 = min(wl.rows, r0 + chunk)
        wf = torch.from_numpy(wl.weight_block(r0, r1)).to(dev)
        qg.qgemv_quantize_weights_rows(wl.wtype, wf, w0, wl.rows, wl.cols, r0, r1 - r0)
        del wf
    ws_list, copies, _keep = weight_copies(w0, wbytes, args.warm)
    rot = itertools.count()           # each launch takes the next copy, in every phase

    x = torch.from_numpy(wl.activations()).to(dev)
    xq = torch.empty((wl.nvec, wl.cols), dtype=torch.int8, device=dev)
    xd = torch.empty((wl.nvec, wl.cols // 32), dtype=torch.float32, device=dev)
    y = torch.empty((wl.nvec, wl.rows), dtype=torch.float32, device=dev)
    wsb = qg.qgemv_workspace_bytes(wl.wtype, wl.rows, wl.cols, wl.nvec)
    work = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    plan = qg.qgemv_plan_for(wl.wtype, wl.rows, wl.cols, wl.nvec)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def quantize():
        qg.qgemv_quantize_act(x, xq, xd, wl.cols, wl.nvec)

    def gemv(i):
        qg.qgemv_batch(wl.wtype, ws_list[next(rot) % copies], xq, xd, y, wl.rows, wl.cols,
                       wl.nvec, workspace=work)

    def step(i):
        qg.qgemv_fused(wl.wtype, ws_list[next(rot) % copies], x, y, wl.rows, wl.cols, wl.nvec,
                       xq_out=xq, xd_out=xd, workspace=work)

    def two_launch(i):
        quantize()
        gemv(i)

    # The GPU's clocks dip for some 10-20 ms whenever work resumes after an idle stretch of a
    # few ms (launch durations rise by up to 20% and recover), so every host-side preparation
    # (graph capture) is done first and the measured phases then run back to back after the
    # warmup steps.
    # a graph holds its launches' weight pointers: enough launches to cover every copy once
    # (at most 5000), so a replay reads cold weights too
    n_graph = max(args.steps, min(copies, 5000))
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def probe(i):
        qg.qgemv_read_probe(ws_list[next(rot) % copies], sink, blocks=4096, nbytes=wbytes)

    graphs = {} if args.counters else {
        name: capture(fn, n_graph) for name, fn in (("step", step), ("gemv", gemv),
                                                    ("two", two_launch), ("probe", probe))}
    # first touch of every weight copy (page mappings) before any measured kernel runs
    for _ in range(2):
        for wc in ws_list:
            qg.qgemv_read_probe(wc, sink, blocks=4096, nbytes=wbytes)
    for i in range(args.warmup):
        step(i)
    marks = Marks(qg, dev)
    marks.mark("step, direct launches (HIP events)")
    ms_step, wall_step = timed(step, args.steps)
    marks.mark("gemv, direct launches")
    ms_gemv, _ = timed(gemv, args.steps)
    marks.mark("quantize_act, direct launches")
    ms_quant, _ = timed(lambda i: quantize(), args.steps)
    marks.mark("quantize + gemv, direct launches")
    ms_two, _ = timed(two_launch, args.steps)
    if args.counters:
        ms_step_graph, ms_gemv_graph, ms_two_graph = ms_step, ms_gemv, ms_two
    else:
        marks.mark("step, graph replay (the roofline's launches)")
        ms_step_graph = replay_timed(graphs["step"], n_graph)
        marks.mark("gemv, graph replay")
        ms_gemv_graph = replay_timed(graphs["gemv"], n_graph)
        marks.mark("quantize + gemv, graph replay")
        ms_two_graph = replay_timed(graphs["two"], n_graph)
    marks.mark("step, batches for the distribution")
    step_dist = spread(step, args.steps)
    # the practical read ceiling: a plain streaming read of the same (cold, rotating) copies
    marks.mark("read probe over the weight copies, direct launches")
    ms_probe_direct, _ = timed(probe, args.steps)
    if args.counters:
        ms_probe = ms_probe_direct
    else:
        marks.mark("read probe over the weight copies, graph replay")
        ms_probe = replay_timed(graphs["probe"], n_graph)
    marks.mark("after the measured phases")
    probe_gbs = wbytes / (ms_probe * 1e-3) / 1e9

    # the step's result must be usable: every output finite
    step(0)
    torch.cuda.synchronize()
    if not bool(torch.isfinite(y).all()):
        print("bench.py: the product gave non-finite outputs", file=sys.stderr)
        sys.exit(1)

    nbytes = algorithmic_bytes(wl, wbytes)
    value = nbytes["step"] / (ms_step * 1e-3) / 1e9
    launches = qg.qgemv_fused_launches(wl.wtype, wl.rows, wl.cols, wl.nvec, True)
    route = qg.qgemv_route(wl.wtype, wl.rows, wl.cols, wl.nvec)
    # the dominant kernel: the step itself when it is one launch, else its GEMV launch; its
    # duration is the mean over a graph replay of back-to-back launches (HIP events around the
    # replay on its stream), which for short kernels excludes the host's per-call time that
    # direct launches from Python add between kernels
    rk_bytes, rk_ms = ((nbytes["step"], ms_step_graph) if launches == 1
                       else (nbytes["gemv"], ms_gemv_graph))
    achieved = rk_bytes / (rk_ms * 1e-3) / 1e9
    kname = roofline_kernel(wl.wtype, plan, wl.nvec, launches, route)
    traffic = load_traffic(args.workload, kname)
    out = {
        "metric": "achieved HBM GB/s and % of roofline, Q4_K GEMV batch-1 (us per GEMV)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8x" + wl.wtype,
        "data": "synthetic",
        "config": {"workload": "%s GEMV W %dx%d, batch %d, cold weights (%d rotating copies, "
                               "%.0f MB)" % (FORMAT_NAMES[wl.wtype], wl.rows, wl.cols, wl.nvec,
                                             copies, copies * wbytes / 1e6),
                   "name": wl.name, "rows": wl.rows, "cols": wl.cols, "nvec": wl.nvec,
                   "weight_bytes": wbytes, "route": route,
                   "plan": plan if route == "vector" else None},
        "us_per_step": round(ms_step * 1e3, 3),
        "us_per_gemv": round(ms_gemv * 1e3, 3),
        "us_per_quantize_act": round(ms_quant * 1e3, 3),
        "us_per_step_two_launch": round(ms_two * 1e3, 3),
        "graph_replay": {"us_per_step": round(ms_step_graph * 1e3, 3),
                         "step_gbs": round(nbytes["step"] / (ms_step_graph * 1e-3) / 1e9, 1),
                         "us_per_gemv": round(ms_gemv_graph * 1e3, 3),
                         "us_per_step_two_launch": round(ms_two_graph * 1e3, 3)},
        "pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "wall_ms_per_step": round(wall_step, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": kname,
                     "algorithmic_bytes_per_launch": rk_bytes, "us_per_launch": round(rk_ms * 1e3, 3),
                     "statistic": "mean launch time over a graph replay of %d back-to-back "
                                  "launches (HIP events on the replay stream); the trace "
                                  "window '%s' holds the same launches" % (
                                      n_graph, "step, graph replay (the roofline's launches)"
                                      if launches == 1 else "gemv, graph replay")},
        "step_launches": launches,
        "us_per_step_distribution": step_dist,
        "read_probe": {"gbs": round(probe_gbs, 1), "us": round(ms_probe * 1e3, 3),
                       "statistic": "graph replay, as for the roofline",
                       "us_direct_launches": round(ms_probe_direct * 1e3, 3),
                       "roofline_achieved_pct_of_probe": round(100 * achieved / probe_gbs, 2)},
        "setup_s": round(setup_s, 1),
        "trace_windows": marks.names,
    }
    if args.traffic_calibration:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for i in range(10):
            qg.qgemv_read_probe(ws_list[i % copies], sink, blocks=4096, nbytes=wbytes)
        src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["traffic_calibration"] = {"read_probe_bytes": wbytes, "copy_bytes": CALIB_COPY_BYTES}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, y.cpu().numpy())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
