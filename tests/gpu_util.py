"""Helpers for the GPU parity tests (device placement, tolerances)."""
from __future__ import annotations

import numpy as np
import pytest

# GEMV / unit-op tolerance: |got - ref| <= ATOL + RTOL * |ref| elementwise
# (fp32 accumulation against the fp64 oracle).
ATOL, RTOL = 1e-4, 2e-3


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(got, ref, atol=ATOL, rtol=RTOL, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    excess = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    i = int(np.argmax(excess))
    assert excess[i] <= 0, (f"{what}: index {i} got {got[i]!r} ref {ref[i]!r} "
                            f"(|diff| {abs(got[i] - ref[i]):.3e}, allowed {atol + rtol * abs(ref[i]):.3e})")
