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

Alongside, in the same JSON line: the Q8_0 GEMV at 4096x4096 ("q8_0_gemv",
the small configuration), Q5_K GEMV at the two Llama-70B FFN shapes
("q5_k_gemv"), and the batched verify pass of self-speculative decoding
("verify_gemm": k = 8 vectors per weight read), and whole-matrix
dequantization to fp32 ("dequant"), each timed like the sweep's per-kernel
times.  Decode measurements ("decode"): the Llama-3-8B-shaped Q8_0
model (128 greedy tokens from position 1024), the Llama-70B-shaped Q4_K/Q6_K
model (64 tokens from 4096), each replayed from a captured HIP graph, the 70B
all-Q6_K model with 24 GiB of layers resident and the rest streamed from
pinned host RAM, and the same with the last --file-layers layers read from a
file each step (the third tier), each as tok/s against the weight-bytes /
8 TB/s bound (or the measured pinned H2D and file read rates).

Flags: --gpus N (only 1 is supported: this path runs on one GPU),
--steps K, --warmup W, --no-cpu-baseline, --cpu-seconds S, --decode
none|8b|70b|all, --stream-tokens T, --file-layers F, --file-dir D.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "achieved HBM GB/s of dequant-GEMV and batch-1 decode tok/s (% of roofline)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--decode", choices=["none", "8b", "70b", "all"], default="all",
                    help="decode measurements: none, the 8B-shaped model, the resident 70B-shaped model, "
                         "or all (8B, 70B, 70B streamed)")
    ap.add_argument("--stream-tokens", type=int, default=3)
    ap.add_argument("--file-layers", type=int, default=8,
                    help="layers of the 70B Q6_K model read from a file each step in the three-tier leg (0: skip)")
    ap.add_argument("--file-dir", default=None, help="directory for the layer file (default: the temp directory)")
    return ap.parse_args()


def gemv_bytes(qtype: int, rows: int, cols: int, nt) -> int:
    """Algorithmic bytes of one GEMV launch: packed weights + x + y."""
    return rows * nt.row_bytes(qtype, cols) + 4 * cols + 4 * rows


def kernel_source_hash() -> str:
    """Hash of the GEMV kernel sources (gemv.hip and the helpers it uses), the
    key under which the committed traffic counters were taken."""
    from block_quantized_decode_dequant_amd import profsum
    return profsum.gemv_source_hash()


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


ONE_GIB = 1 << 30


def copies_for(nbytes: int) -> int:
    """Copies of a matrix so that consecutive reads of one copy are at least
    1 GiB of reads apart (4x the 256 MB last-level cache)."""
    return max(2, -(-ONE_GIB // nbytes) + 1)


def time_rotated(torch, call, n_copies: int, steps: int, side) -> float:
    """Mean microseconds per launch of call(copy): two HIP graphs of `steps`
    launches each (a warm-up and a timed one) walk one continuous cyclic
    sequence of copy indices, so two reads of one copy are always n_copies
    launches apart, across the two replays too.  Events bracket the timed
    replay on the stream the kernels run on."""
    graphs = []
    with torch.cuda.stream(side):
        call(0)                                   # first use outside capture
        for start in (0, steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for i in range(start, start + steps):
                    call(i % n_copies)
            graphs.append(g)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(side):
        graphs[0].replay()
        a.record(side)
        graphs[1].replay()
        b.record(side)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    del graphs
    return us


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


def read_ceiling(nt, torch, dev, nbytes=4 << 30, reps=20):
    """Measured HBM read ceiling (GB/s): a vectorized read-and-reduce kernel
    over 4 GiB, best of 20 launches, each timed with events on its stream."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4096, dtype=torch.float32, device=dev)
    best = 0.0
    for r in range(reps + 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        nt.nt_read_bytes(buf, nbytes, sink)
        b.record()
        torch.cuda.synchronize()
        if r >= 2:
            best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return round(best, 1)


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

    # The W warmup steps and the K timed steps are each captured as one HIP
    # graph (step s runs its eight launches on weight copy s mod copies) and
    # replayed once, so the timed region holds exactly K steps of kernels with
    # no host work or per-step graph launch between them (replaying one
    # eight-launch graph per step from the host added ~17 us per step).
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step(0)                                   # first use outside capture
        g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        if args.warmup > 0:
            with torch.cuda.graph(g_warm, stream=side):
                for i in range(args.warmup):
                    step(i)
        with torch.cuda.graph(g_timed, stream=side):
            for s_ in range(args.steps):
                step(args.warmup + s_)            # continues the warm-up's copy rotation
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        if args.warmup > 0:
            g_warm.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    with torch.cuda.stream(side):
        g_timed.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graphs = [g_warm, g_timed]
    step_bytes = sum(c["bytes"] for c in cases)
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9

    # Per-kernel durations, measured live: each case launched back to back
    # `steps` times from a captured graph, one pair of events around the
    # replay on the launch stream (no host work between the kernels).  Each
    # case rotates copies of its own matrix sized so that two reads of one
    # copy are at least 1 GiB of reads apart, so the last-level cache cannot
    # serve them (the sweep's own copies are sized for the whole step).
    per_case_ms = []
    for c in cases:
        n = copies_for(c["bytes"])
        Ws = list(c["W"]) + [c["W"][0].clone() for _ in range(max(0, n - len(c["W"])))]
        us = time_rotated(torch, lambda i: nt.nt_gemv(c["qt"], Ws[i], c["x"], c["y"], c["rows"], c["cols"]),
                          n, args.steps, side)
        per_case_ms.append(us * 1e-3)
        c["case_copies"] = n
        del Ws
        torch.cuda.empty_cache()
    case_sum_ms = sum(per_case_ms)

    # per-kernel totals; a kernel is one instantiation (block type, path, tile
    # rows), as the library reports it, which is what rocprofv3 lists by name
    kern = {}
    for c, ms in zip(cases, per_case_ms):
        li = nt.nt_gemv_launch_info(c["qt"], c["rows"], c["cols"])
        k = f"gemv {c['type']} lds vec{li['vec']}" if li["fast"] else f"gemv {c['type']} generic"
        a = kern.setdefault(k, dict(bytes=0, ms=0.0, launches=0))
        a["bytes"] += c["bytes"]
        a["ms"] += ms
        a["launches"] += 1
    dom = max(kern, key=lambda k: kern[k]["ms"])
    d = kern[dom]
    achieved = d["bytes"] / (d["ms"] * 1e-3) / 1e9
    traffic = load_traffic(dom)
    ceiling = read_ceiling(nt, torch, dev)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": dom, "bytes_per_launch": d["bytes"] // d["launches"],
                "avg_launch_us": round(d["ms"] / d["launches"] * 1e3, 3),
                "read_ceiling": ceiling, "frac_of_read_ceiling": round(achieved / ceiling, 4)}
    detail = [dict(type=c["type"], rows=c["rows"], cols=c["cols"], bytes=c["bytes"],
                   launch=nt.nt_gemv_launch_info(c["qt"], c["rows"], c["cols"]), copies=c["case_copies"],
                   us=round(ms * 1e3, 3), gbs=round(c["bytes"] / (ms * 1e-3) / 1e9, 1),
                   frac=round(c["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
              for c, ms in zip(cases, per_case_ms)]
    del graphs
    for c in cases:
        del c["W"]
    torch.cuda.empty_cache()
    return dict(value=value, ms_per_step=ms_per_step, roofline=roofline, detail=detail,
                copies=copies, step_bytes=step_bytes, case_sum_ms=case_sum_ms)


def q8_0_gemv(steps):
    """The single Q8_0 GEMV workload, y = W x with W 4096 x 4096: int8 codes
    uniform on [-127, 127], one fp16 scale |N(0,1)| * 0.01 per 32-value block,
    x ~ N(0, 1), seed 0 (synth.q8_0_random_matrix, drawn on the host), timed
    like the sweep's per-kernel times with copies >= 1 GiB apart.  Reported
    beside the sweep, not part of `value`."""
    import torch

    from block_quantized_decode_dequant_amd import nt, synth, workloads

    dev = torch.device("cuda:0")
    wl = workloads.Q8_0_GEMV
    rows, cols = wl["rows"], wl["cols"]
    base = torch.from_numpy(synth.q8_0_random_matrix(workloads.SEED, rows, cols)).to(dev)
    x = torch.from_numpy(synth.activation(workloads.SEED, synth.Q8_CFG_X, cols)).to(dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    nbytes = base.numel()
    copies = copies_for(nbytes)
    Ws = [base] + [base.clone() for _ in range(copies - 1)]
    side = torch.cuda.Stream()
    us = time_rotated(torch, lambda i: nt.nt_gemv(nt.Q8_0, Ws[i], x, y, rows, cols), copies, steps, side)
    alg = gemv_bytes(nt.Q8_0, rows, cols, nt)
    li = nt.nt_gemv_launch_info(nt.Q8_0, rows, cols)
    out = {"workload": wl["name"], "rows": rows, "cols": cols, "bytes": alg, "copies": copies, "launch": li,
           "us": round(us, 3), "gbs": round(alg / (us * 1e-6) / 1e9, 1),
           "frac": round(alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del Ws, base
    torch.cuda.empty_cache()
    return out


def q5_k_gemv(steps):
    """Q5_K GEMV at the two Llama-70B FFN projection shapes (28672x8192 and
    8192x28672), measured like the sweep's per-kernel times: weights encoded
    on the device from the sweep's N(0, 0.02) values, rotated copies (>= 1 GiB
    apart), one HIP graph of `steps` back-to-back launches, events around its
    replay.  Reported beside the sweep, not part of `value`."""
    import torch

    from block_quantized_decode_dequant_amd import nt, synth, workloads

    dev = torch.device("cuda:0")
    out = []
    for si in (2, 3):
        rows, cols = workloads.KQ_SHAPES[si]
        w32 = torch.from_numpy(synth.normal_f32(workloads.SEED, workloads.kq_w_stream(si), rows * cols,
                                                std=0.02)).to(dev)
        x = torch.from_numpy(synth.activation(workloads.SEED, workloads.kq_x_stream(si), cols)).to(dev)
        nbytes = rows * nt.row_bytes(nt.Q5_K, cols)
        base = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        nt.nt_quantize(nt.Q5_K, w32, base, rows * cols)
        del w32
        copies = copies_for(nbytes)
        Ws = [base] + [base.clone() for _ in range(copies - 1)]
        y = torch.empty(rows, dtype=torch.float32, device=dev)
        side = torch.cuda.Stream()
        us = time_rotated(torch, lambda i: nt.nt_gemv(nt.Q5_K, Ws[i], x, y, rows, cols), copies, steps, side)
        alg = nbytes + 4 * cols + 4 * rows
        out.append({"rows": rows, "cols": cols, "bytes": alg, "us": round(us, 3),
                    "gbs": round(alg / (us * 1e-6) / 1e9, 1), "frac": round(alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)})
        del Ws, base
        torch.cuda.empty_cache()
    return out


DEQUANT_CASES = [("q8_0", 4096, 4096), ("q4_k", 8192, 8192), ("q6_k", 8192, 8192)]


def dequant_leg(steps):
    """nt_dequant of whole matrices to fp32 (the Q8_0 4096x4096 and 70B
    8192x8192 K-quant projection shapes), timed like the sweep: blocks encoded
    on the device from N(0, 0.02) values, block copies and output buffers each
    rotated over at least 1 GiB, one HIP graph of `steps` launches.  "bytes":
    blocks read + fp32 output written; "fill_gbs": the same outputs written by
    a plain fill (torch's fill_), the write-side ceiling.  Reported beside the
    sweep, not part of `value`."""
    import math

    import torch

    from block_quantized_decode_dequant_amd import nt, synth, workloads

    dev = torch.device("cuda:0")
    out = []
    for name, rows, cols in DEQUANT_CASES:
        t = {"q8_0": nt.Q8_0, "q4_k": nt.Q4_K, "q6_k": nt.Q6_K}[name]
        n = rows * cols
        w32 = torch.from_numpy(synth.normal_f32(workloads.SEED, 800 + rows // 1024, n, std=0.02)).to(dev)
        nbytes = rows * nt.row_bytes(t, cols)
        base = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        nt.nt_quantize(t, w32, base, n)
        del w32
        Ws = [base] + [base.clone() for _ in range(copies_for(nbytes) - 1)]
        Ys = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(copies_for(4 * n))]
        cyc = len(Ws) * len(Ys) // math.gcd(len(Ws), len(Ys))
        side = torch.cuda.Stream()
        us = time_rotated(torch, lambda i: nt.nt_dequant(t, Ws[i % len(Ws)], Ys[i % len(Ys)], n), cyc, steps, side)
        fill_us = time_rotated(torch, lambda i: Ys[i % len(Ys)].fill_(1.0), len(Ys), steps, side)
        alg = nbytes + 4 * n
        out.append({"type": name, "rows": rows, "cols": cols, "bytes": alg, "us": round(us, 3),
                    "gbs": round(alg / (us * 1e-6) / 1e9, 1), "frac": round(alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "fill_gbs": round(4 * n / (fill_us * 1e-6) / 1e9, 1)})
        del Ws, Ys, base
        torch.cuda.empty_cache()
    return out


VERIFY_K = 8
VERIFY_CASES = [("q8_0", 4096, 4096), ("q4_k", 8192, 8192), ("q4_k", 28672, 8192), ("q6_k", 8192, 8192),
                ("q6_k", 8192, 28672)]


def verify_gemm(steps):
    """The batched verify pass (nt_gemm_batch, k = 8 draft tokens against one
    matrix) at the 8B Q8_0 and 70B K-quant projection shapes, timed like the
    sweep (device-encoded weights from N(0, 0.02) values, rotated copies
    >= 1 GiB apart, one HIP graph of `steps` launches) beside one GEMV of the
    same matrix.  "gbs": algorithmic bytes (weights once, k activation and
    output vectors) per second; "x_vs_k_gemv": k GEMV times over the batched
    time.  Reported beside the sweep, not part of `value`."""
    import numpy as np
    import torch

    from block_quantized_decode_dequant_amd import nt, synth, workloads

    dev = torch.device("cuda:0")
    k = VERIFY_K
    out = []
    for name, rows, cols in VERIFY_CASES:
        t = {"q8_0": nt.Q8_0, "q4_k": nt.Q4_K, "q6_k": nt.Q6_K}[name]
        w32 = torch.from_numpy(synth.normal_f32(workloads.SEED, 700 + rows // 1024 + cols // 1024, rows * cols,
                                                std=0.02)).to(dev)
        X = torch.from_numpy(np.concatenate([synth.activation(workloads.SEED, 710 + n, cols)
                                             for n in range(k)])).to(dev)
        nbytes = rows * nt.row_bytes(t, cols)
        base = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        nt.nt_quantize(t, w32, base, rows * cols)
        del w32
        copies = copies_for(nbytes)
        Ws = [base] + [base.clone() for _ in range(copies - 1)]
        Y = torch.empty(k * rows, dtype=torch.float32, device=dev)
        nws = nt.nt_gemm_batch_workspace_bytes(t, rows, cols)
        ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
        side = torch.cuda.Stream()
        us = time_rotated(torch, lambda i: nt.nt_gemm_batch(t, Ws[i], X, Y, rows, cols, k, ws), copies, steps, side)
        us1 = time_rotated(torch, lambda i: nt.nt_gemv(t, Ws[i], X[:cols], Y[:rows], rows, cols), copies, steps,
                           side)
        alg = nbytes + 4 * k * (cols + rows)
        out.append({"type": name, "rows": rows, "cols": cols, "k": k, "bytes": alg, "us": round(us, 3),
                    "gbs": round(alg / (us * 1e-6) / 1e9, 1), "frac": round(alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "gemv_us": round(us1, 3), "x_vs_k_gemv": round(k * us1 / us, 2)})
        del Ws, base
        torch.cuda.empty_cache()
    return out


def time_decode(model, shape, n_tokens, warmup=8):
    import torch
    dev = torch.device("cuda:0")
    side = torch.cuda.Stream()
    d_tok = torch.tensor([1], dtype=torch.int32, device=dev)
    d_pos = torch.tensor([shape.ctx], dtype=torch.int32, device=dev)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device=dev)

    def run(n):
        with torch.cuda.stream(side):
            for _ in range(n):
                model.step(d_tok, d_pos, logits, d_tok)

    run(warmup)
    torch.cuda.synchronize()
    d_pos.fill_(shape.ctx)
    d_tok.fill_(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(n_tokens)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(d_pos.item()) == shape.ctx + n_tokens
    return wall


def decode_resident(shape):
    import torch

    from block_quantized_decode_dequant_amd import devmodel

    t0 = time.perf_counter()
    model, extra = devmodel.build(shape)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    wall = time_decode(model, shape, shape.n_tokens)
    tps = shape.n_tokens / wall
    wbytes = devmodel.weight_bytes_per_token(shape)
    kv_mid = devmodel.kv_bytes_per_token(shape, shape.ctx + shape.n_tokens // 2)
    bound = PEAK_HBM_GBS * 1e9 / wbytes
    bound_kv = PEAK_HBM_GBS * 1e9 / (wbytes + kv_mid)
    out = {"tok_s": round(tps, 2), "ms_per_token": round(wall / shape.n_tokens * 1e3, 4),
           "tokens": shape.n_tokens, "start_pos": shape.ctx, "weight_bytes_per_token": wbytes,
           "bound_tok_s": round(bound, 1), "frac_of_bound": round(tps / bound, 4),
           "bound_with_kv_tok_s": round(bound_kv, 1), "frac_of_bound_with_kv": round(tps / bound_kv, 4),
           "achieved_gbs": round((wbytes + kv_mid) * tps / 1e9, 1), "graph": True,
           "build_s": round(build_s, 1)}
    model.close()
    del model, extra
    torch.cuda.empty_cache()
    return out


def pinned_h2d_ceiling(nbytes=1 << 30, reps=5):
    import torch
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    best = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        d.copy_(h, non_blocking=True)
        torch.cuda.synchronize()
        best = max(best, nbytes / (time.perf_counter() - t0) / 1e9)
    del h, d
    return best


def decode_streamed(shape, cap_bytes=24 << 30, n_tokens=3):
    import torch

    from block_quantized_decode_dequant_amd import devmodel, nt

    types = devmodel.tensor_types(shape.weights)
    cfg = nt.model_config(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                          shape.ffn, shape.vocab, shape.ctx_cap, shape.rms_eps, shape.rope_theta)
    _, blob = nt.nt_layer_blob_layout(cfg, [types[n] for n in devmodel.MATS])
    first = min(shape.n_layers, cap_bytes // blob)
    ceiling = pinned_h2d_ceiling()
    t0 = time.perf_counter()
    model, extra = devmodel.build(shape, streamed_from=first)
    blobs, nbytes = devmodel.fill_streamed_blobs(shape, first)
    build_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    dbuf = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    copy_stream = torch.cuda.Stream()
    model.stream_layers(first, blobs, dbuf[0], dbuf[1], copy_stream)
    d_tok = torch.tensor([1], dtype=torch.int32, device=dev)
    d_pos = torch.tensor([shape.ctx], dtype=torch.int32, device=dev)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        model.step(d_tok, d_pos, logits, d_tok)           # warm-up token
    torch.cuda.synchronize()
    walls, copies, comps = [], [], []
    t0 = time.perf_counter()
    for _ in range(n_tokens):
        with torch.cuda.stream(side):
            model.step(d_tok, d_pos, logits, d_tok)
        st = model.stream_stats()
        walls.append(st["wall_ms"])
        copies.append(st["copy_ms"])
        comps.append(st["compute_ms"])
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    ns = shape.n_layers - first
    h2d = ns * nbytes
    copy_ms, comp_ms, wall_ms = (sum(v) / len(v) for v in (copies, comps, walls))
    out = {"resident_layers": int(first), "streamed_layers": int(ns), "blob_bytes": int(nbytes),
           "h2d_bytes_per_token": int(h2d), "tok_s": round(n_tokens / total, 3),
           "ms_per_token": round(total / n_tokens * 1e3, 2),
           "h2d_gbs": round(h2d / (copy_ms * 1e-3) / 1e9, 2),
           "h2d_gbs_wall": round(h2d / (wall_ms * 1e-3) / 1e9, 2),
           "pinned_h2d_ceiling_gbs": round(ceiling, 2),
           "frac_of_h2d_ceiling": round(h2d / (copy_ms * 1e-3) / 1e9 / ceiling, 4),
           "bound_tok_s": round(ceiling * 1e9 / h2d, 3),
           "copy_ms": round(copy_ms, 2), "streamed_compute_ms": round(comp_ms, 2), "wall_ms": round(wall_ms, 2),
           "compute_hidden_frac": round(max(0.0, min(1.0, (copy_ms + comp_ms - wall_ms) / comp_ms)), 4)
           if comp_ms > 0 else None,
           "tokens": n_tokens, "cap_bytes": int(cap_bytes), "build_s": round(build_s, 1)}
    model.stream_layers(None, None, None, None, None)
    model.close()
    del model, extra, blobs, dbuf
    torch.cuda.empty_cache()
    return out


def host_cpu():
    """CPU model name, logical CPUs the OS reports and CPUs this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


CPU_SHARE = 16      # host threads one single-GPU job may keep busy on the GPU machines


def oracle_decode_token(threads: int):
    """Seconds the oracle takes for one decode token of the Llama-3-8B-shaped
    Q8_0 model (32 layers, full 128256-row head, attention over 1024 cached
    positions).  The weights are all-zero Q8_0 blocks: the oracle decodes and
    multiplies every block whatever its values, so its time per token does not
    depend on them; the KV prefix is seeded N(0, 1) fp16."""
    import numpy as np

    import oracle as O
    from block_quantized_decode_dequant_amd import synth, workloads

    s = workloads.LLAMA_8B_Q8_0
    H, D, F, V = s.hidden, s.head_dim, s.ffn, s.vocab
    QD, KD = s.n_q_heads * D, s.n_kv_heads * D
    z = lambda r, c: O.QTensor(O.Q8_0, np.zeros(r * O.row_bytes(O.Q8_0, c), np.uint8))
    ones = np.ones(H, np.float32)
    layers = [O.LayerWeights(attn_norm=ones, wq=z(QD, H), wk=z(KD, H), wv=z(KD, H), wo=z(H, QD), ffn_norm=ones,
                             w_gate=z(F, H), w_up=z(F, H), w_down=z(H, F)) for _ in range(s.n_layers)]
    w = O.ModelWeights(tok_embd=z(V, H), output_norm=ones, output=z(V, H), layers=layers)
    cfg = O.Config(s.n_layers, H, s.n_q_heads, s.n_kv_heads, D, F, V, s.ctx_cap, s.rms_eps, s.rope_theta)
    kk = np.stack([synth.kv_prefix_bits(0, l, 0, s.n_kv_heads, s.ctx_cap, D, s.ctx) for l in range(s.n_layers)])
    vv = np.stack([synth.kv_prefix_bits(0, l, 1, s.n_kv_heads, s.ctx_cap, D, s.ctx) for l in range(s.n_layers)])
    dec = O.Decoder(cfg, w, kk, vv)
    t0 = time.perf_counter()
    dec.step(1, s.ctx, nthreads=threads)
    return time.perf_counter() - t0


def decode_file_tier(shape, n_file, where=None, vram_cap=24 << 30, n_tokens=2):
    """The three-tier mode on the 70B all-Q6_K model: the first 24 GiB of
    layers resident, the last n_file layers read from a file every step
    (O_DIRECT when the file system allows it) through two pinned staging
    buffers, the layers between them from pinned host RAM; reads, copies and
    compute are pipelined by the host (a copy is enqueued once its read has
    finished).  The file holds only the file tier's layers; it is written
    first, then read back, then deleted."""
    import shutil
    import tempfile

    import torch

    from block_quantized_decode_dequant_amd import devmodel, nt

    types = devmodel.tensor_types(shape.weights)
    tl = [types[n] for n in devmodel.MATS]
    cfg = nt.model_config(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                          shape.ffn, shape.vocab, shape.ctx_cap, shape.rms_eps, shape.rope_theta)
    _, blob = nt.nt_layer_blob_layout(cfg, tl)
    stride = -(-blob // 4096) * 4096
    where = where or tempfile.gettempdir()
    free = shutil.disk_usage(where).free
    n_file = int(min(n_file, max(0, (free - (4 << 30)) // stride)))   # leave 4 GiB free on the disk
    if n_file <= 0:
        return {"skipped": f"no room for one {stride}-byte layer in {where} ({free} bytes free)"}
    first_streamed = int(min(shape.n_layers, vram_cap // blob))
    first_file = shape.n_layers - n_file
    planned = nt.nt_tier_plan(cfg, tl, vram_cap, (first_file - first_streamed) * blob)
    assert planned == (first_streamed, first_file), planned
    t0 = time.perf_counter()
    model, extra = devmodel.build(shape, streamed_from=first_streamed)
    blobs, nbytes = devmodel.fill_streamed_blobs(shape, first_streamed, last=first_file)
    fd, path = tempfile.mkstemp(prefix="nt_layers_", suffix=".bin", dir=where)
    os.close(fd)
    try:
        tw = time.perf_counter()
        stride_w, _ = devmodel.write_streamed_file(shape, first_file, path)
        os.sync()
        write_s = time.perf_counter() - tw
        build_s = time.perf_counter() - t0
        dev = torch.device("cuda:0")
        dbuf = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
        raw = torch.empty(2 * stride + 4096, dtype=torch.uint8, pin_memory=True)
        lead = (-raw.data_ptr()) % 4096
        st0, st1 = raw[lead:lead + stride], raw[lead + stride:lead + 2 * stride]
        copy_stream = torch.cuda.Stream()
        model.stream_layers_tiered(first_streamed, blobs, dbuf[0], dbuf[1], copy_stream, path, first_file, 0,
                                   stride_w, st0, st1, direct=True)
        d_tok = torch.tensor([1], dtype=torch.int32, device=dev)
        d_pos = torch.tensor([shape.ctx], dtype=torch.int32, device=dev)
        logits = torch.empty(shape.vocab, dtype=torch.float32, device=dev)
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            model.step(d_tok, d_pos, logits, d_tok)           # warm-up token
        torch.cuda.synchronize()
        recs = []
        t1 = time.perf_counter()
        for _ in range(n_tokens):
            with torch.cuda.stream(side):
                model.step(d_tok, d_pos, logits, d_tok)
            recs.append((model.stream_stats(), model.file_stats()))
        torch.cuda.synchronize()
        total = time.perf_counter() - t1
        avg = lambda f: sum(f(r) for r in recs) / len(recs)
        read_ms = avg(lambda r: r[1]["read_ms"])
        span_ms = avg(lambda r: r[1]["read_span_ms"])
        copy_ms = avg(lambda r: r[0]["copy_ms"])
        comp_ms = avg(lambda r: r[0]["compute_ms"])
        wall_ms = avg(lambda r: r[0]["wall_ms"])
        fbytes = n_file * nbytes
        ns = shape.n_layers - first_streamed
        out = {"resident_layers": first_streamed, "pinned_layers": first_file - first_streamed,
               "file_layers": n_file, "blob_bytes": int(nbytes), "file_stride": int(stride_w),
               "o_direct": bool(recs[-1][1]["direct"]), "file_dir": where,
               "file_bytes_per_token": int(fbytes), "h2d_bytes_per_token": int(ns * nbytes),
               "tok_s": round(n_tokens / total, 3), "ms_per_token": round(total / n_tokens * 1e3, 1),
               "file_read_gbs": round(fbytes / (read_ms * 1e-3) / 1e9, 2),
               "file_read_gbs_span": round(fbytes / (span_ms * 1e-3) / 1e9, 2),
               "h2d_gbs": round(ns * nbytes / (copy_ms * 1e-3) / 1e9, 2),
               "read_ms": round(read_ms, 1), "read_span_ms": round(span_ms, 1), "copy_ms": round(copy_ms, 1),
               "streamed_compute_ms": round(comp_ms, 2), "wall_ms": round(wall_ms, 1),
               "copy_and_compute_hidden_frac": round(max(0.0, min(1.0, (span_ms + copy_ms + comp_ms - wall_ms)
                                                                 / (copy_ms + comp_ms))), 4),
               "tokens": n_tokens, "write_s": round(write_s, 1), "build_s": round(build_s, 1)}
        model.stream_layers(None, None, None, None, None)
        model.close()
        del model, extra, blobs, dbuf, raw
        torch.cuda.empty_cache()
        return out
    finally:
        os.unlink(path)


def cpu_baseline(seconds: float):
    """The oracle's fp64 GEMV on the first rows of every sweep matrix, on
    CPU_SHARE threads and on one core; and one oracle decode token of the
    8B-shaped model on one core."""
    import numpy as np

    import oracle as O
    from block_quantized_decode_dequant_amd import synth, workloads

    model, n_logical, n_usable = host_cpu()
    cores = min(CPU_SHARE, n_usable)
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

    def timed(nthreads, budget):
        done_bytes, t0, passes = 0, time.perf_counter(), 0
        while True:
            for t, blocks, r, cols, x, nbytes in work:
                O.gemv(t, blocks, r, cols, x, nthreads=nthreads)
                done_bytes += nbytes
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return done_bytes / el / 1e9, passes, el

    gbs, passes, el = timed(cores, seconds)
    gbs1, passes1, el1 = timed(1, max(1.0, seconds / 4))
    tok1 = oracle_decode_token(1)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"first {sample_rows} rows of each of the 8 sweep matrices, "
                      f"{passes} passes, {el:.1f} s, fp64 oracle GEMV with {cores} threads; "
                      f"one core: {passes1} passes, {el1:.1f} s",
            "value_one_core": round(gbs1, 3),
            "cpu_model": model, "logical_cpus": n_logical, "usable_cpus": n_usable,
            "threads_note": f"{cores} threads: the host share of one single-GPU job",
            "decode_8b_token_s_one_core": round(tok1, 2),
            "decode_8b_token_sample": "one token of the Llama-3-8B-shaped Q8_0 model at position 1024 "
                                      "(32 layers, 128256-row head), oracle on one core; all-zero weight "
                                      "blocks (the oracle's work does not depend on the values)"}


def done(what: str, t0: float):
    """One line on stderr as each leg ends (the JSON line stays the only stdout)."""
    print(f"bench.py: {what} done ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)


def main():
    args = parse()
    t0 = time.perf_counter()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(no sharding or collectives are built)", file=sys.stderr)
        raise SystemExit(2)
    g = run_gpu(args)
    done("sweep", t0)
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
        "per_case_sum_ms": round(g["case_sum_ms"], 4),
        "roofline": g["roofline"],
        "detail": g["detail"],
    }
    line["q8_0_gemv"] = q8_0_gemv(args.steps)
    line["q5_k_gemv"] = q5_k_gemv(args.steps)
    line["verify_gemm"] = verify_gemm(args.steps)
    line["dequant"] = dequant_leg(args.steps)
    done("q8_0, q5_k, verify and dequant legs", t0)
    if args.decode != "none":
        dec = {}
        if args.decode in ("8b", "all"):
            dec["llama3_8b_q8_0"] = decode_resident(workloads.LLAMA_8B_Q8_0)
            done("8B decode", t0)
        if args.decode in ("70b", "all"):
            dec["llama70b_q4_k_q6_k"] = decode_resident(workloads.LLAMA_70B_MIX)
            done("70B decode", t0)
        if args.decode == "all":
            dec["llama70b_q6_k_streamed_24gib"] = decode_streamed(workloads.LLAMA_70B_Q6K,
                                                                  n_tokens=args.stream_tokens)
            done("70B streamed decode", t0)
            if args.file_layers > 0:
                dec["llama70b_q6_k_three_tier_file"] = decode_file_tier(workloads.LLAMA_70B_Q6K, args.file_layers,
                                                                        args.file_dir)
                done("70B three-tier decode", t0)
        line["decode"] = dec
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        done("cpu baseline", t0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
