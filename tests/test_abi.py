"""The C-ABI library loads, exports every call include/nt.h declares, and
rejects bad arguments before touching the GPU.  CPU-only: nothing here
launches a kernel.  Calls that pass placeholder addresses run only on hosts
with no GPU, where the library must stop at NT_ENODEV.
"""
import ctypes as C
import os
import re

import pytest

from block_quantized_decode_dequant_amd import nt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nt.h")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="placeholder addresses are only passed "
                                 "on hosts without a GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nt_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_call():
    L = C.CDLL(nt.lib_path())
    names = declared_functions()
    assert len(names) >= 18
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_version_status_and_geometry():
    L = nt.lib()
    assert L.nt_abi_version() == 2
    for s in range(8):
        assert nt.status_str(s).startswith("NT_")
    assert [L.nt_qtype_block_elems(t) for t in (nt.Q8_0, nt.Q4_0, nt.Q4_K, nt.Q6_K)] == [32, 32, 256, 256]
    assert [L.nt_qtype_block_bytes(t) for t in (nt.Q8_0, nt.Q4_0, nt.Q4_K, nt.Q6_K)] == [34, 18, 144, 210]
    assert nt.row_bytes(nt.Q6_K, 8192) == 32 * 210
    assert nt.row_bytes(nt.Q8_0, 4096) == 128 * 34
    assert nt.row_bytes(nt.Q4_K, 300) == -1
    assert L.nt_qtype_block_elems(99) == -1


A = 0x10000     # placeholder, 16-byte aligned; never dereferenced


def _gemv(t, W, x, y, rows, cols, acc=0):
    return nt.lib().nt_gemv(t, C.c_void_p(W), C.c_void_p(x), C.c_void_p(y), rows, cols, acc, None)


@no_gpu_only
def test_gemv_argument_errors():
    assert _gemv(nt.Q4_K, 0, A, A, 4, 256) == nt.NT_EINVAL
    assert "null" in nt.last_error()
    assert _gemv(nt.Q4_K, A, A, A, 4, 100) == nt.NT_ESHAPE
    assert _gemv(nt.Q8_0, A, A, A, -1, 64) == nt.NT_EINVAL
    assert _gemv(nt.Q8_0, A, A, A, 4, 65536 + 32) == nt.NT_ESHAPE
    assert _gemv(nt.Q8_0, A + 2, A, A, 4, 64) == nt.NT_EALIGN
    assert _gemv(nt.Q8_0, A, A + 4, A, 4, 64) == nt.NT_EALIGN
    assert _gemv(5, A, A, A, 4, 64) == nt.NT_EINVAL
    assert _gemv(nt.Q8_0, 0, 0, 0, 0, 64) == nt.NT_OK        # nothing to do
    assert _gemv(nt.Q6_K, A, A, A, 4, 256) == nt.NT_ENODEV   # valid, but no GPU here


def _batch(t, W, X, Y, rows, cols, k, ws=A, ws_bytes=4 << 20):
    return nt.lib().nt_gemm_batch(t, C.c_void_p(W), C.c_void_p(X), C.c_void_p(Y), rows, cols, k, 0,
                                  C.c_void_p(ws), ws_bytes, None)


@no_gpu_only
def test_gemm_batch_argument_errors():
    wsb = nt.nt_gemm_batch_workspace_bytes
    # 16384 bytes of split counters, then one activation record per 256
    # columns where a first kernel writes them (8192 bytes of split
    # activations, 512 of sub-block sums for K-quants with mins, 32 of
    # scales; none where the main kernel forms them in LDS), then, when the
    # columns are split between workgroups, fp32 partial sums of 8 vectors
    # per column range
    rec = {nt.Q4_K: 8736, nt.Q5_K: 8736, nt.Q6_K: 8224, nt.Q8_0: 8224, nt.Q4_0: 8224}
    C = 16384
    assert wsb(nt.Q4_0, 1, 32) == C + 8224          # one range, records from the first kernel
    assert wsb(nt.Q8_0, 1, 32) == C                 # one range, records formed in LDS
    for t, rows, cols in [(nt.Q4_K, 8192, 8192), (nt.Q6_K, 8192, 28672), (nt.Q8_0, 4096, 4096),
                          (nt.Q4_K, 3, 65536), (nt.Q5_K, 40040, 2048), (nt.Q4_0, 600, 8960)]:
        ns = -(-cols // 256)
        extra = wsb(t, rows, cols) - C
        for records in (0, ns * rec[t]):
            split, r = divmod(extra - records, 8 * rows * 4)
            if extra >= records and r == 0 and split != 1 and split <= min(ns, 64):
                break
        else:
            raise AssertionError((t, rows, cols, extra))
    assert wsb(nt.Q8_0, 4096, 4096) == C + 16 * 8224             # records from the first kernel, no split
    assert wsb(nt.Q4_K, 28672, 8192) == C + 2 * 8 * 28672 * 4   # records in LDS, two-way split
    assert wsb(nt.Q4_K, 1500, 5888) == C + 8 * 8 * 1500 * 4     # records in LDS, eight-way split
    assert wsb(nt.Q4_K, 3, 65536) > C + 3 * 8 * 4 * 2   # a few rows: split between workgroups
    assert wsb(nt.F32, 4, 256) == 0 and wsb(nt.Q4_K, 4, 100) == 0 and wsb(nt.Q4_K, 4, 65536 + 256) == 0
    assert wsb(nt.Q4_K, -1, 256) == 0
    assert _batch(nt.Q4_K, A, A, A, 4, 256, 0) == nt.NT_EINVAL
    assert _batch(nt.Q4_K, A, A, A, 4, 256, 9) == nt.NT_EINVAL
    assert _batch(nt.F32, A, A, A, 4, 256, 2) == nt.NT_EINVAL
    assert _batch(nt.F16, A, A, A, 4, 256, 2) == nt.NT_EINVAL
    assert _batch(nt.Q4_0, A, A, A, 4, 96, 2) == nt.NT_ENODEV           # valid (3 blocks), but no GPU here
    assert _batch(nt.Q4_K, A, A, A, 4, 100, 2) == nt.NT_ESHAPE
    assert _batch(nt.Q8_0, A, A, A, 4, 65536 + 32, 2) == nt.NT_ESHAPE
    assert _batch(nt.Q4_K, A, A, A, -1, 256, 2) == nt.NT_EINVAL
    assert _batch(nt.Q4_K, 0, A, A, 4, 256, 2) == nt.NT_EINVAL
    assert _batch(nt.Q4_K, A, A, A, 4, 2048, 2, ws=0) == nt.NT_EINVAL        # needs a workspace
    assert _batch(nt.Q4_K, A, A, A, 4, 256, 2, ws=0) == nt.NT_EINVAL
    assert _batch(nt.Q4_K, A + 4, A, A, 4, 256, 2) == nt.NT_EALIGN
    assert _batch(nt.Q4_K, A, A + 4, A, 4, 256, 2) == nt.NT_EALIGN
    assert _batch(nt.Q4_K, A, A, A + 2, 4, 256, 2) == nt.NT_EALIGN
    assert _batch(nt.Q4_K, A, A, A, 4, 256, 2, ws=A + 8) == nt.NT_EALIGN
    assert _batch(nt.Q4_K, A, A, A, 4, 2048, 2, ws_bytes=wsb(nt.Q4_K, 4, 2048) - 4) == nt.NT_ENOMEM
    assert _batch(nt.Q4_K, 0, 0, 0, 0, 256, 2, ws=0) == nt.NT_OK          # nothing to do
    assert _batch(nt.Q6_K, A, A, A + 4, 4, 256, 8) == nt.NT_ENODEV        # valid, but no GPU here


def _multi(t, Ws, rows, ys, cols, x=A, gain=None, eps=1e-5, acc=0):
    k = len(Ws)
    W = (C.c_void_p * k)(*Ws)
    r = (C.c_int64 * k)(*rows)
    y = (C.c_void_p * k)(*ys)
    return nt.lib().nt_gemv_multi(t, k, W, r, y, cols, C.c_void_p(x), C.c_void_p(gain), eps, acc, None)


def _swiglu(t, Wg, Wu, rows, cols, x=A, gain=None, h=A, eps=1e-5):
    return nt.lib().nt_gemv_swiglu(t, C.c_void_p(Wg), C.c_void_p(Wu), rows, cols, C.c_void_p(x),
                                   C.c_void_p(gain), eps, C.c_void_p(h), None)


@no_gpu_only
def test_fused_gemv_argument_errors():
    assert _multi(nt.Q4_K, [A, A], [4, 4], [A, A], 2048) == nt.NT_ENODEV     # valid
    assert _multi(nt.Q4_K, [], [], [], 2048) == nt.NT_EINVAL                 # nseg 0
    assert _multi(nt.Q4_K, [A] * 4, [1] * 4, [A] * 4, 2048) == nt.NT_EINVAL  # nseg 4
    assert _multi(nt.Q4_K, [A], [4], [A], 300) == nt.NT_ESHAPE
    assert _multi(nt.Q6_K, [A], [4], [A], 256) == nt.NT_ESHAPE               # 210-byte rows
    assert _multi(nt.Q8_0, [A], [4], [A], 65536) == nt.NT_ESHAPE             # too wide for the fused path
    assert _multi(nt.Q4_K, [A + 4], [4], [A], 2048) == nt.NT_EALIGN
    assert _multi(nt.Q4_K, [A], [4], [A], 2048, gain=A + 4) == nt.NT_EALIGN
    assert _multi(nt.Q4_K, [0], [4], [A], 2048) == nt.NT_EINVAL
    assert _multi(nt.Q4_K, [A], [-1], [A], 2048) == nt.NT_EINVAL
    assert _multi(nt.Q4_K, [A], [4], [A], 2048, eps=-1.0) == nt.NT_EINVAL
    assert _multi(nt.Q4_K, [A], [0], [A], 2048) == nt.NT_OK                 # nothing to do
    assert _swiglu(nt.Q8_0, A, A, 64, 4096) == nt.NT_ENODEV                 # valid
    assert _swiglu(nt.Q8_0, A, 0, 64, 4096) == nt.NT_EINVAL
    assert _swiglu(nt.Q6_K, A, A, 64, 256) == nt.NT_ESHAPE
    assert _swiglu(nt.Q8_0, A, A, 64, 4096, h=A + 8) == nt.NT_EALIGN
    assert _swiglu(nt.Q8_0, A, A, 0, 4096) == nt.NT_OK


def test_launch_info_reports_the_copy_width():
    assert nt.nt_gemv_launch_info(nt.Q4_K, 8192, 8192)["vec"] == 16
    assert nt.nt_gemv_launch_info(nt.Q6_K, 8192, 8192)["vec"] == 16
    assert nt.nt_gemv_launch_info(nt.Q6_K, 64, 1536)["vec"] == 4      # 1260-byte rows
    assert nt.nt_gemv_launch_info(nt.Q8_0, 64, 320)["vec"] == 4       # 340-byte rows
    assert not nt.nt_gemv_launch_info(nt.Q6_K, 64, 256)["fast"]       # 210-byte rows
    assert not nt.nt_gemv_launch_info(nt.Q8_0, 8, 40960)["fast"]      # wider than 32768


@no_gpu_only
def test_dequant_and_calibration_argument_errors():
    L = nt.lib()
    v = C.c_void_p
    assert L.nt_dequant(nt.Q4_0, v(A), v(A), 33, None) == nt.NT_ESHAPE
    assert L.nt_dequant(nt.Q4_0, v(A + 8), v(A), 32, None) == nt.NT_EALIGN
    assert L.nt_dequant(nt.Q4_0, v(A), v(A + 2), 32, None) == nt.NT_EALIGN
    assert L.nt_dequant(nt.F32, v(A), v(A), 32, None) == nt.NT_EINVAL
    assert L.nt_dequant_q6_k(v(0), v(A), 256, None) == nt.NT_EINVAL
    assert L.nt_dequant_q8_0(v(A), v(A), 0, None) == nt.NT_OK
    assert L.nt_dequant_q8_0(v(A), v(A), 64, None) == nt.NT_ENODEV
    assert L.nt_read_bytes(v(A), 24, v(A), None) == nt.NT_ESHAPE
    assert L.nt_copy_bytes(v(A), v(A + 4), 32, None) == nt.NT_EALIGN


def test_binding_refuses_host_tensors():
    import torch
    W = torch.zeros(34 * 2, dtype=torch.uint8)
    x = torch.zeros(64)
    y = torch.zeros(1)
    with pytest.raises(ValueError, match="GPU tensor"):
        nt.nt_gemv_q8_0(W, x, y, 1, 64)


@no_gpu_only
def test_op_argument_errors():
    L = nt.lib()
    v = C.c_void_p
    assert L.nt_rmsnorm(v(A), v(A), v(A), -1, 1e-5, None) == nt.NT_EINVAL
    assert L.nt_rmsnorm(v(A), v(0), v(A), 8, 1e-5, None) == nt.NT_EINVAL
    assert L.nt_rmsnorm(v(A + 2), v(A), v(A), 8, 1e-5, None) == nt.NT_EALIGN
    assert L.nt_rope(v(A), v(A), 4, 2, 63, v(A), 1e4, None) == nt.NT_ESHAPE
    assert L.nt_rope(v(A), v(A), 4, 2, 64, v(0), 1e4, None) == nt.NT_EINVAL
    assert L.nt_softmax(v(0), 5, None) == nt.NT_EINVAL
    assert L.nt_swiglu(v(A), v(A), v(A + 1), 5, None) == nt.NT_EALIGN
    assert L.nt_argmax(v(A), 0, v(A), None) == nt.NT_EINVAL
    assert L.nt_embed(nt.Q4_K, v(A), 10, 100, v(A), v(A), None) == nt.NT_ESHAPE
    assert L.nt_embed(nt.Q4_K, v(A + 4), 10, 256, v(A), v(A), None) == nt.NT_EALIGN
    assert L.nt_rmsnorm(v(A), v(A), v(A), 8, 1e-5, None) == nt.NT_ENODEV


@no_gpu_only
def test_attention_argument_errors():
    L = nt.lib()
    v = C.c_void_p
    good = nt.attn_desc(32, 8, 128, 1152)
    ws = nt.nt_attn_workspace_bytes(good)
    assert ws == 32 * 32 * 130 * 4      # chunk 36 -> 32 chunks of (max, sum, o[128]) per q head
    args = lambda d, wsb=ws, kn=A: (C.byref(d), v(A), v(kn), v(kn), v(A), v(A), v(A), v(A), v(A), wsb, None)
    assert L.nt_attn_decode(*args(nt.attn_desc(12, 8, 128, 64))) == nt.NT_ESHAPE     # 12 % 8 != 0
    assert L.nt_attn_decode(*args(nt.attn_desc(32, 8, 96, 64))) == nt.NT_ESHAPE      # head_dim 96
    assert L.nt_attn_decode(*args(nt.attn_desc(48, 3, 64, 64))) == nt.NT_ESHAPE      # group of 16
    assert L.nt_attn_decode(*args(nt.attn_desc(32, 8, 128, 0))) == nt.NT_EINVAL
    assert L.nt_attn_decode(*args(good, ws - 4)) == nt.NT_ENOMEM
    assert L.nt_attn_decode(C.byref(good), v(A), v(A), v(0), v(A), v(A), v(A), v(A), v(A), ws, None) == nt.NT_EINVAL
    assert L.nt_attn_decode(*args(good)) == nt.NT_ENODEV
    assert L.nt_attn_decode(*args(good, ws, 0)) == nt.NT_ENODEV      # both NULL is allowed
    assert L.nt_attn_decode(*args(nt.attn_desc(32, 8, 128, 1152, rope_theta=-1.0))) == nt.NT_EINVAL
    assert L.nt_attn_decode(*args(nt.attn_desc(32, 8, 128, 1152, rope_theta=5e5))) == nt.NT_ENODEV
    assert L.nt_attn_decode(C.byref(good), v(A + 4), v(A), v(A), v(A), v(A), v(A), v(A), v(A), ws,
                            None) == nt.NT_EALIGN                     # q must be 16-byte aligned
    assert nt.nt_attn_workspace_bytes(nt.attn_desc(32, 8, 96, 64)) == 0


def test_tier_plan_fills_vram_then_pinned_then_file():
    """The data-path choice (VRAM, then pinned host RAM, then the file) as
    plain arithmetic over whole layer blobs."""
    cfg = nt.model_config(80, 8192, 64, 8, 128, 28672, 128256, 4160)
    types = [nt.Q6_K] * 7
    _, blob = nt.nt_layer_blob_layout(cfg, types)
    assert blob == 701890560                       # the write-up's ~670 MB (MiB) per 70B layer
    assert nt.nt_tier_plan(cfg, types, 24 << 30, 0) == (36, 36)            # 24 GiB resident, the rest from the file
    assert nt.nt_tier_plan(cfg, types, 24 << 30, 10 * blob + 5) == (36, 46)
    assert nt.nt_tier_plan(cfg, types, 0, 1 << 50) == (0, 80)
    assert nt.nt_tier_plan(cfg, types, 1 << 50, 1 << 50) == (80, 80)
    assert nt.nt_tier_plan(cfg, types, blob - 1, blob) == (0, 1)
