#!/usr/bin/env python3
"""Benchmark: achieved HBM bandwidth of the fused dequantize-GEMV kernels.

One step = one pass over the K-quant GEMV sweep on the Llama-70B projection
shapes (8192x8192, 1024x8192, 28672x8192, 8192x28672, each in Q4_K and Q6_K:
eight launches), with weights already resident in HBM.  Every step uses a
different copy of each matrix (copies rotated so that at least 1 GiB of weights
lies between two reads of the same copy), so reads come from HBM and not from
the 256 MB last-level cache.  `value` is the step's algorithmic bytes over its
time.  Each launch is bracketed by HIP events on the stream it runs on; the
kernel with the most time in the timed region gives the `roofline` object.

The CPU baseline times the oracle (plain fp64 C, test-side code) on a bounded
sample of the same workload: the first rows of each matrix.

Flags: --gpus N (only 1 is supported: this path runs on one GPU),
--steps K, --warmup W, --no-cpu-baseline, --decode (also time the
Llama-8B-shaped decode, when the library provides it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "achieved HBM GB/s of dequant-GEMV and batch-1 decode tok/s (% of roofline)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_traffic.json")
GEMV_SRC = os.path.join(ROOT, "block_quantized_decode_dequant_amd", "csrc", "gemv.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--decode", action="store_true")
    return ap.parse_args()


def gemv_bytes(qtype: int, rows: int, cols: int, nt) -> int:
    """Algorithmic bytes of one GEMV launch: packed weights + x + y."""
    return rows * nt.row_bytes(qtype, cols) + 4 * cols + 4 * rows


def kernel_source_hash() -> str:
    return hashlib.sha256(open(GEMV_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("gemv_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("per_launch_bytes", {}).get(kernel)


def build_sweep(nt, torch, dev, synth, workloads):
    """Device-resident sweep: for each (type, shape) R rotated copies of the
    encoded matrix, plus x and y."""
    cases = []
    for si, (rows, cols) in enumerate(workloads.KQ_SHAPES):
        w32 = torch.from_numpy(synth.normal_f32(workloads.SEED, workloads.kq_w_stream(si),
                                                rows * cols, std=0.02)).to(dev)
        x = torch.from_numpy(synth.activation(workloads.SEED, workloads.kq_x_stream(si), cols)).to(dev)
        for tname in workloads.KQ_TYPES:
            qt = nt.QTYPES[tname]
            nbytes = rows * nt.row_bytes(qt, cols)
            base = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            nt.nt_quantize(qt, w32, base, rows * cols)
            cases.append(dict(type=tname, qt=qt, rows=rows, cols=cols, x=x, base=base,
                              y=torch.empty(rows, dtype=torch.float32, device=dev),
                              bytes=gemv_bytes(qt, rows, cols, nt)))
        del w32
    step_bytes = sum(c["bytes"] for c in cases)
    copies = max(2, -(-(1 << 30) // step_bytes) + 1)   # >= 1 GiB between reuses
    for c in cases:
        c["W"] = [c["base"]] + [c["base"].clone() for _ in range(copies - 1)]
        del c["base"]
    torch.cuda.synchronize()
    return cases, copies


def run_gpu(args):
    import torch

    from block_quantized_decode_dequant_amd import nt, synth, workloads

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    nt.lib()
    cases, copies = build_sweep(nt, torch, dev, synth, workloads)

    def step(i, events=None):
        for j, c in enumerate(cases):
            if events is not None:
                events[j][0].record()
            nt.nt_gemv(c["qt"], c["W"][i % copies], c["x"], c["y"], c["rows"], c["cols"])
            if events is not None:
                events[j][1].record()

    # One HIP graph per weight copy, each holding one step (eight launches),
    # so the timed region replays steps with no host work between kernels.
    graphs = []
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for i in range(args.warmup):
            step(i)
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step(i)
            graphs.append(g)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for s in range(args.steps):
        graphs[s % copies].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_bytes = sum(c["bytes"] for c in cases)
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9

    # Per-kernel durations, measured live: the same steps launched directly,
    # queued behind a short delay kernel so that every launch is already
    # waiting on the stream and each event pair brackets one kernel.
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in cases] for _ in range(args.steps)]
    torch.cuda.synchronize()
    nt.nt_delay(min(1e6, 2000.0 + 400.0 * args.steps))
    for s in range(args.steps):
        step(s, ev[s])
    torch.cuda.synchronize()
    per_case_ms = [sum(ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(args.steps)) / args.steps
                   for j in range(len(cases))]
    span_ms = ev[0][0][0].elapsed_time(ev[-1][-1][1]) / args.steps

    # per-kernel (one kernel per block type) totals
    kern = {}
    for c, ms in zip(cases, per_case_ms):
        k = f"gemv {c['type']}"
        a = kern.setdefault(k, dict(bytes=0, ms=0.0, launches=0))
        a["bytes"] += c["bytes"]
        a["ms"] += ms
        a["launches"] += 1
    dom = max(kern, key=lambda k: kern[k]["ms"])
    d = kern[dom]
    achieved = d["bytes"] / (d["ms"] * 1e-3) / 1e9
    traffic = load_traffic(dom)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": dom, "bytes_per_launch": d["bytes"] // d["launches"],
                "avg_launch_us": round(d["ms"] / d["launches"] * 1e3, 3)}
    detail = [dict(type=c["type"], rows=c["rows"], cols=c["cols"], bytes=c["bytes"],
                   us=round(ms * 1e3, 3), gbs=round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
                   frac=round(c["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
              for c, ms in zip(cases, per_case_ms)]
    del graphs
    for c in cases:
        del c["W"]
    torch.cuda.empty_cache()
    return dict(value=value, ms_per_step=ms_per_step, roofline=roofline, detail=detail,
                copies=copies, step_bytes=step_bytes, queued_step_ms=span_ms)


def cpu_baseline(seconds: float):
    """The oracle's fp64 GEMV on the first rows of every sweep matrix."""
    import numpy as np

    import oracle as O
    from block_quantized_decode_dequant_amd import synth, workloads

    cores = O.default_threads()
    sample_rows = 256
    work = []
    for si, (rows, cols) in enumerate(workloads.KQ_SHAPES):
        r = min(rows, sample_rows)
        w = synth.normal_f32(workloads.SEED, workloads.kq_w_stream(si), r * cols, std=0.02)
        x = synth.activation(workloads.SEED, workloads.kq_x_stream(si), cols).astype(np.float64)
        for tname in workloads.KQ_TYPES:
            t = O.QTYPES[tname]
            blocks = O.quantize(t, w)
            work.append((t, blocks, r, cols, x, r * O.row_bytes(t, cols) + 4 * cols + 4 * r))
    done_bytes, t0, passes = 0, time.perf_counter(), 0
    while True:
        for t, blocks, r, cols, x, nbytes in work:
            O.gemv(t, blocks, r, cols, x, nthreads=cores)
            done_bytes += nbytes
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done_bytes / el / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"first {sample_rows} rows of each of the 8 sweep matrices, "
                      f"{passes} passes, {el:.1f} s, fp64 oracle GEMV with {cores} threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(no sharding or collectives are built)", file=sys.stderr)
        raise SystemExit(2)
    g = run_gpu(args)
    from block_quantized_decode_dequant_amd import workloads

    line = {
        "metric": METRIC,
        "value": round(g["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "K-quant dequant-GEMV sweep, Llama-70B projection shapes",
                   "shapes": workloads.KQ_SHAPES, "types": workloads.KQ_TYPES,
                   "weights": "fp32 N(0,0.02) encoded in HBM, x N(0,1), seed 0",
                   "rotated_copies": g["copies"], "step_bytes": g["step_bytes"]},
        "frac_of_peak": round(g["value"] / PEAK_HBM_GBS, 4),
        "queued_launch_ms_per_step": round(g["queued_step_ms"], 4),
        "roofline": g["roofline"],
        "detail": g["detail"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
