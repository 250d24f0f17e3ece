"""Summaries of rocprofv3 CSV output for the profiles/ directory.

    python -m block_quantized_decode_dequant_amd.profsum stats KERNEL_STATS.csv [--top N]
    python -m block_quantized_decode_dequant_amd.profsum trace KERNEL_TRACE.csv --match SUBSTR
    python -m block_quantized_decode_dequant_amd.profsum pertoken KERNEL_TRACE.csv [--skip N]
    python -m block_quantized_decode_dequant_amd.profsum traffic --fetch F.csv --write W.csv \
        --cal-fetch CF.csv --cal-write CW.csv --cal-bytes N --out JSON

`traffic` turns FETCH_SIZE / WRITE_SIZE readings (KiB per dispatch) into HBM
bytes per launch of each GEMV kernel instantiation.  The counters are scaled
by what they read for the plain copy kernel of known size (N bytes read and N
written) in a calibration run, so the result is in true bytes.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# the GEMV kernels' sources: the kernel file and the copy and wait helpers it uses
GEMV_SRCS = [os.path.join(HERE, "csrc", "gemv.hip"), os.path.join(HERE, "csrc", "device_util.h")]


def gemv_source_hash() -> str:
    """First 16 hex digits of the SHA-256 of the GEMV kernel sources, in order."""
    h = hashlib.sha256()
    for path in GEMV_SRCS:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]

FMT = {"F80": "q8_0", "F40": "q4_0", "F4K": "q4_k", "F5K": "q5_k", "F6K": "q6_k"}


def kernel_key(name: str):
    """The benchmark's name for a GEMV kernel instantiation, or None."""
    m = re.search(r"gemv_lds<nt::\(anonymous namespace\)::(F\w+), (\d+), (true|false)(?:, (true|false))?>", name)
    if m:
        # both activation layouts under one name, as the benchmark groups them
        return f"gemv {FMT[m.group(1)]} lds vec{m.group(2)}" + (" +norm" if m.group(3) == "true" else "")
    if "gemv_generic" in name:
        return "gemv generic"
    return None


def short(name: str, n=96) -> str:
    name = name.replace("nt::(anonymous namespace)::", "")
    name = re.sub(r"\(.*\)$", "", name)
    return name if len(name) <= n else name[: n - 3] + "..."


def cmd_stats(a):
    rows = list(csv.DictReader(open(a.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print(f"{'kernel':60s} {'calls':>7s} {'avg_us':>10s} {'total_ms':>10s} {'%':>6s}")
    for r in rows[: a.top]:
        print(f"{short(r['Name'], 60):60s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.3f} "
              f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}")


def trace_durations(path: str):
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        out[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def cmd_trace(a):
    for name, d in sorted(trace_durations(a.csv).items()):
        if a.match in name:
            k = kernel_key(name) or short(name, 60)
            print(f"{k:40s} n={len(d):5d} avg_us={sum(d) / len(d):9.3f} min_us={min(d):9.3f} max_us={max(d):9.3f}")


def cmd_pertoken(a):
    """Per-token time of a decode run: the trace between embedding launches
    (one per token), after --skip warm-up tokens, by kernel and launch shape."""
    rows = list(csv.DictReader(open(a.csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    idx = [i for i, r in enumerate(rows) if "embed_kernel" in r["Kernel_Name"]]
    skip = min(a.skip, len(idx) - 2)
    seg = rows[idx[skip]:idx[-1]]
    ntok = len(idx) - 1 - skip
    wall = (int(seg[-1]["Start_Timestamp"]) - int(seg[0]["Start_Timestamp"])) / 1e3
    per, cnt = collections.defaultdict(float), collections.Counter()
    busy, gaps, prev_end = 0.0, 0.0, None
    for r in seg:
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        key = (short(r["Kernel_Name"], 44), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
               int(r["Workgroup_Size_X"]))
        per[key] += (e - s) / 1e3
        cnt[key] += 1
        busy += (e - s) / 1e3
        if prev_end is not None:
            gaps += max(0, s - prev_end) / 1e3
        prev_end = e
    print(f"tokens {ntok}: wall {wall / ntok:.1f} us/token, kernel time {busy / ntok:.1f} us/token, "
          f"idle gaps {gaps / ntok:.1f} us/token, {len(seg) / ntok:.1f} launches/token")
    print(f"{'kernel':44s} {'wg.x':>6s} {'thr':>5s} {'n/tok':>6s} {'avg_us':>8s} {'us/token':>9s} {'%':>6s}")
    for k, v in sorted(per.items(), key=lambda kv: -kv[1]):
        print(f"{k[0]:44s} {k[1]:6d} {k[2]:5d} {cnt[k] / ntok:6.1f} {v / cnt[k]:8.2f} {v / ntok:9.1f} "
              f"{100 * v / busy:6.2f}")


def counter_by_kernel(path: str, counter: str):
    """Average counter value (summed over instances) per dispatch, by kernel name."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def cmd_traffic(a):
    cf = counter_by_kernel(a.cal_fetch, "FETCH_SIZE")
    cw = counter_by_kernel(a.cal_write, "WRITE_SIZE")
    copy = [k for k in cf if "copy_kernel" in k]
    if not copy:
        raise SystemExit("no copy_kernel dispatch in the calibration run")
    kib_f, _ = cf[copy[0]]
    kib_w, _ = cw[copy[0]]
    scale_f = a.cal_bytes / (kib_f * 1024.0)
    scale_w = a.cal_bytes / (kib_w * 1024.0)
    f = counter_by_kernel(a.fetch, "FETCH_SIZE")
    w = counter_by_kernel(a.write, "WRITE_SIZE")
    # instantiations the benchmark groups under one name (both activation
    # layouts) are pooled: per-launch bytes = their total over their dispatches
    tot = collections.defaultdict(lambda: [0.0, 0.0, 0])
    for name, (kib, n) in f.items():
        key = kernel_key(name)
        if not key or key == "gemv generic":
            continue
        wkib = w.get(name, (0.0, 0))[0]
        tot[key][0] += kib * n
        tot[key][1] += wkib * n
        tot[key][2] += n
    per_launch, detail = {}, {}
    for key, (kib_sum, wkib_sum, n) in tot.items():
        kib, wkib = kib_sum / n, wkib_sum / n
        per_launch[key] = round(kib * 1024 * scale_f + wkib * 1024 * scale_w)
        detail[key] = {"dispatches": n, "fetch_kib_raw": round(kib, 1), "write_kib_raw": round(wkib, 1),
                       "fetch_bytes": round(kib * 1024 * scale_f), "write_bytes": round(wkib * 1024 * scale_w)}
    rec = {"gemv_source_sha256_16": gemv_source_hash(),
           "calibration": {"kernel": "copy_kernel", "bytes_each_way": a.cal_bytes,
                           "fetch_kib_raw": round(kib_f, 1), "write_kib_raw": round(kib_w, 1),
                           "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4)},
           "per_launch_bytes": per_launch, "detail": detail}
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--top", type=int, default=25)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--match", default="gemv")
    pt = sub.add_parser("pertoken")
    pt.add_argument("csv")
    pt.add_argument("--skip", type=int, default=1)
    r = sub.add_parser("traffic")
    for k in ("fetch", "write", "cal_fetch", "cal_write", "out"):
        r.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    r.add_argument("--cal-bytes", type=int, default=1 << 28)
    a = ap.parse_args()
    {"stats": cmd_stats, "trace": cmd_trace, "pertoken": cmd_pertoken, "traffic": cmd_traffic}[a.cmd](a)


if __name__ == "__main__":
    main()
