"""Runs the plain copy and read kernels at known sizes (for counter calibration).

    python -m block_quantized_decode_dequant_amd.calib_run [--copy-bytes N] [--read-bytes N]

Under `rocprofv3 --pmc FETCH_SIZE` (or WRITE_SIZE) the copy kernel's reading
gives the factor between the counter and true bytes: it moves exactly N bytes
each way.
"""
import argparse

import torch

from . import nt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--copy-bytes", type=int, default=1 << 28)
    ap.add_argument("--read-bytes", type=int, default=1 << 30)
    ap.add_argument("--reps", type=int, default=5)
    a = ap.parse_args()
    dev = torch.device("cuda:0")
    src = torch.empty(max(a.copy_bytes, a.read_bytes), dtype=torch.uint8, device=dev)
    dst = torch.empty(a.copy_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.float32, device=dev)
    for _ in range(a.reps):
        nt.nt_copy_bytes(dst, src, a.copy_bytes)
        nt.nt_read_bytes(src, a.read_bytes, sink)
    torch.cuda.synchronize()
    print(f"copy {a.copy_bytes} B x{a.reps}, read {a.read_bytes} B x{a.reps}", flush=True)


if __name__ == "__main__":
    main()
