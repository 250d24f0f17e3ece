"""Thin ctypes binding over libnt.so (the C ABI declared in include/nt.h).

Argument marshalling only: each function takes torch tensors (device memory)
or raw integer addresses, checks that tensors live on the GPU and are large
enough for what the call will touch, and passes plain pointers and sizes to
the library.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  If libnt.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os

from . import build as _build

NT_OK, NT_EINVAL, NT_ESHAPE, NT_EALIGN, NT_ENOMEM, NT_EHIP, NT_ESTATE, NT_ENODEV = range(8)
F32, F16, Q4_0, Q8_0, Q4_K, Q6_K = 0, 1, 2, 8, 12, 14
QTYPES = {"f32": F32, "f16": F16, "q4_0": Q4_0, "q8_0": Q8_0, "q4_k": Q4_K, "q6_k": Q6_K}
BLOCK_ELEMS = {Q8_0: 32, Q4_0: 32, Q4_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 144, Q6_K: 210}


class NTError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func}: status {status}: {message}")
        self.status = status


_lib = None


def lib_path() -> str:
    return _build.LIB_PATH


def lib():
    """Load libnt.so.  It must have been built (``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libnt.so not found at {path}; build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = C.CDLL(path)
        _declare(L)
        _lib = L
    return _lib


def _declare(L):
    vp, i64, i32, st = C.c_void_p, C.c_int64, C.c_int, C.c_int
    sig = {
        "nt_abi_version": (i32, []),
        "nt_status_str": (C.c_char_p, [st]),
        "nt_last_error": (C.c_char_p, []),
        "nt_qtype_block_elems": (i64, [i32]),
        "nt_qtype_block_bytes": (i64, [i32]),
        "nt_qtype_row_bytes": (i64, [i32, i64]),
        "nt_dequant": (st, [i32, vp, vp, i64, vp]),
        "nt_gemv": (st, [i32, vp, vp, vp, i64, i64, i32, vp]),
        "nt_quantize": (st, [i32, vp, vp, i64, vp]),
        "nt_read_bytes": (st, [vp, i64, vp, vp]),
        "nt_copy_bytes": (st, [vp, vp, i64, vp]),
        "nt_delay": (st, [C.c_double, vp]),
    }
    for t in ("q8_0", "q4_0", "q4_k", "q6_k"):
        sig[f"nt_dequant_{t}"] = (st, [vp, vp, i64, vp])
        sig[f"nt_gemv_{t}"] = (st, [vp, vp, vp, i64, i64, i32, vp])
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


# ---- marshalling helpers ------------------------------------------------------
def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _ptr(t, need_bytes: int = 0, name: str = "buffer"):
    """Device address of a torch tensor (checked) or a raw integer address."""
    if t is None:
        return None
    if isinstance(t, int):
        return C.c_void_p(t)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < need_bytes:
        raise ValueError(f"{name} holds {have} bytes, the call touches {need_bytes}")
    return C.c_void_p(t.data_ptr())


def _check(status: int, func: str):
    if status != NT_OK:
        msg = lib().nt_last_error().decode(errors="replace")
        raise NTError(status, func, msg)


def row_bytes(qtype: int, cols: int) -> int:
    return lib().nt_qtype_row_bytes(qtype, cols)


def abi_version() -> int:
    return lib().nt_abi_version()


def status_str(s: int) -> str:
    return lib().nt_status_str(s).decode()


def last_error() -> str:
    return lib().nt_last_error().decode(errors="replace")


# ---- dequant ---------------------------------------------------------------------
def nt_dequant(qtype: int, blocks, out, n: int, stream=None):
    be, bb = BLOCK_ELEMS.get(qtype, 1), BLOCK_BYTES.get(qtype, 1)
    _check(lib().nt_dequant(qtype, _ptr(blocks, n // be * bb, "blocks"), _ptr(out, 4 * n, "out"),
                            n, _stream(stream)), "nt_dequant")


def nt_dequant_q8_0(blocks, out, n, stream=None): nt_dequant(Q8_0, blocks, out, n, stream)
def nt_dequant_q4_0(blocks, out, n, stream=None): nt_dequant(Q4_0, blocks, out, n, stream)
def nt_dequant_q4_k(blocks, out, n, stream=None): nt_dequant(Q4_K, blocks, out, n, stream)
def nt_dequant_q6_k(blocks, out, n, stream=None): nt_dequant(Q6_K, blocks, out, n, stream)


# ---- GEMV --------------------------------------------------------------------------
def nt_gemv(qtype: int, W, x, y, rows: int, cols: int, accumulate: bool = False, stream=None):
    rb = row_bytes(qtype, cols)
    need_w = rows * rb if rb > 0 else 0
    _check(lib().nt_gemv(qtype, _ptr(W, need_w, "W"), _ptr(x, 4 * cols, "x"), _ptr(y, 4 * rows, "y"),
                         rows, cols, int(bool(accumulate)), _stream(stream)), "nt_gemv")


def nt_gemv_q8_0(W, x, y, rows, cols, accumulate=False, stream=None): nt_gemv(Q8_0, W, x, y, rows, cols, accumulate, stream)
def nt_gemv_q4_0(W, x, y, rows, cols, accumulate=False, stream=None): nt_gemv(Q4_0, W, x, y, rows, cols, accumulate, stream)
def nt_gemv_q4_k(W, x, y, rows, cols, accumulate=False, stream=None): nt_gemv(Q4_K, W, x, y, rows, cols, accumulate, stream)
def nt_gemv_q6_k(W, x, y, rows, cols, accumulate=False, stream=None): nt_gemv(Q6_K, W, x, y, rows, cols, accumulate, stream)


# ---- encode -----------------------------------------------------------------------------
def nt_quantize(qtype: int, x, blocks, n: int, stream=None):
    be, bb = BLOCK_ELEMS.get(qtype, 1), BLOCK_BYTES.get(qtype, 1)
    _check(lib().nt_quantize(qtype, _ptr(x, 4 * n, "x"), _ptr(blocks, n // be * bb, "blocks"), n,
                             _stream(stream)), "nt_quantize")


# ---- calibration ---------------------------------------------------------------------
def nt_read_bytes(src, nbytes: int, sink, stream=None):
    _check(lib().nt_read_bytes(_ptr(src, nbytes, "src"), nbytes, _ptr(sink, 4 * 4096, "sink"),
                               _stream(stream)), "nt_read_bytes")


def nt_copy_bytes(dst, src, nbytes: int, stream=None):
    _check(lib().nt_copy_bytes(_ptr(dst, nbytes, "dst"), _ptr(src, nbytes, "src"), nbytes,
                               _stream(stream)), "nt_copy_bytes")


def nt_delay(microseconds: float, stream=None):
    _check(lib().nt_delay(float(microseconds), _stream(stream)), "nt_delay")
