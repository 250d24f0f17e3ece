"""Plain fp64 CPU oracle for quantized batch-1 Llama decode -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never links or
calls it, and it shares no code with the HIP path.

The arithmetic lives in C (``oracle/*.c``, built into ``liboracle.so`` by
``oracle.build``); this module only marshals numpy arrays through ctypes.
Every function cites the passage of the ntransformer write-up (GeekNews
topic 26894) that it follows in the C source it calls.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field

import numpy as np

from . import build as _build

F32, F16, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 0, 1, 2, 8, 12, 13, 14
QTYPES = {"f32": F32, "f16": F16, "q4_0": Q4_0, "q8_0": Q8_0, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K}

_lib = None


def lib():
    """Load liboracle.so, building it first only if it is missing."""
    global _lib
    if _lib is None:
        path = _build.LIB_PATH
        if not os.path.exists(path):
            _build.build_oracle()
        L = C.CDLL(path)
        vp, i64, i32, d = C.c_void_p, C.c_int64, C.c_int, C.c_double
        sig = {
            "or_f16_to_f64": (d, [C.c_uint16]),
            "or_f64_to_f16_rne": (C.c_uint16, [d]),
            "or_f64_to_f16_up": (C.c_uint16, [d]),
            "or_block_elems": (i64, [i32]),
            "or_block_bytes": (i64, [i32]),
            "or_row_bytes": (i64, [i32, i64]),
            "or_dequant": (i32, [i32, vp, i64, vp]),
            "or_quantize": (i32, [i32, vp, i64, vp]),
            "or_pack_q8_0": (i32, [vp, vp, i64, vp]),
            "or_gemv": (i32, [i32, vp, i64, i64, vp, vp, i32]),
            "or_gemv_rows": (i32, [i32, vp, i64, i64, vp, vp, i64, vp, i32]),
            "or_rmsnorm": (None, [vp, vp, i64, d, vp]),
            "or_rope": (None, [vp, i32, i32, i64, d]),
            "or_softmax": (None, [vp, i64, vp]),
            "or_silu": (d, [d]),
            "or_swiglu": (None, [vp, vp, i64, vp]),
            "or_argmax": (i64, [vp, i64]),
            "or_attention": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, d, vp]),
            "or_decode_step": (i32, [vp, vp, vp, vp, C.c_int32, i64, vp, vp, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


# ---- fp16 ------------------------------------------------------------------
def f16_to_f64(h: int) -> float:
    return lib().or_f16_to_f64(int(h))


def f64_to_f16_rne(v: float) -> int:
    return lib().or_f64_to_f16_rne(float(v))


def f64_to_f16_up(v: float) -> int:
    return lib().or_f64_to_f16_up(float(v))


# ---- block formats -----------------------------------------------------------
def block_elems(t: int) -> int:
    return lib().or_block_elems(t)


def block_bytes(t: int) -> int:
    return lib().or_block_bytes(t)


def row_bytes(t: int, cols: int) -> int:
    return lib().or_row_bytes(t, cols)


def dequant(t: int, blocks: np.ndarray, n: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert blocks.size >= n // block_elems(t) * block_bytes(t)
    out = np.empty(n, np.float32)
    _check(lib().or_dequant(t, _ptr(blocks), n, _ptr(out)), "dequant")
    return out


def quantize(t: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    be = block_elems(t)
    out = np.zeros(x.size // be * block_bytes(t), np.uint8)
    _check(lib().or_quantize(t, _ptr(x), x.size, _ptr(out)), "quantize")
    return out


def pack_q8_0(d_bits: np.ndarray, qs: np.ndarray) -> np.ndarray:
    d_bits = np.ascontiguousarray(d_bits, dtype=np.uint16).reshape(-1)
    qs = np.ascontiguousarray(qs, dtype=np.int8).reshape(-1)
    assert qs.size == 32 * d_bits.size
    out = np.empty(34 * d_bits.size, np.uint8)
    _check(lib().or_pack_q8_0(_ptr(d_bits), _ptr(qs), d_bits.size, _ptr(out)), "pack_q8_0")
    return out


# ---- ops -----------------------------------------------------------------------
def gemv(t: int, W: np.ndarray, rows: int, cols: int, x, nthreads: int | None = None) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    assert W.size >= rows * row_bytes(t, cols)
    x = _f64(x)
    assert x.size == cols
    y = np.empty(rows, np.float64)
    _check(lib().or_gemv(t, _ptr(W), rows, cols, _ptr(x), _ptr(y),
                         nthreads or default_threads()), "gemv")
    return y


def gemm_batch(t: int, W: np.ndarray, rows: int, cols: int, X, nthreads: int | None = None) -> np.ndarray:
    """The verify pass of self-speculative decoding (ntransformer write-up,
    "Overview"): k activation vectors against one matrix, Y[n] = W . X[n],
    by its definition, one oracle GEMV per vector.  X: k x cols; returns
    k x rows (fp64)."""
    X = np.atleast_2d(np.asarray(X))
    return np.stack([gemv(t, W, rows, cols, X[n], nthreads) for n in range(X.shape[0])])


def gemv_rows(t: int, W: np.ndarray, rows: int, cols: int, x, row_ids,
              nthreads: int | None = None) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x = _f64(x)
    ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    y = np.empty(ids.size, np.float64)
    _check(lib().or_gemv_rows(t, _ptr(W), rows, cols, _ptr(x), _ptr(ids), ids.size, _ptr(y),
                              nthreads or default_threads()), "gemv_rows")
    return y


def rmsnorm(x, g, eps: float) -> np.ndarray:
    x, g = _f64(x), _f64(g)
    y = np.empty_like(x)
    lib().or_rmsnorm(_ptr(x), _ptr(g), x.size, eps, _ptr(y))
    return y


def rope(v, n_heads: int, head_dim: int, pos: int, theta: float) -> np.ndarray:
    v = _f64(v).copy()
    assert v.size == n_heads * head_dim
    lib().or_rope(_ptr(v), n_heads, head_dim, pos, theta)
    return v


def softmax(s) -> np.ndarray:
    s = _f64(s)
    p = np.empty_like(s)
    lib().or_softmax(_ptr(s), s.size, _ptr(p))
    return p


def silu(a: float) -> float:
    return lib().or_silu(float(a))


def swiglu(g, u) -> np.ndarray:
    g, u = _f64(g), _f64(u)
    out = np.empty_like(g)
    lib().or_swiglu(_ptr(g), _ptr(u), g.size, _ptr(out))
    return out


def argmax(v) -> int:
    v = _f64(v)
    return int(lib().or_argmax(_ptr(v), v.size))


def attention(q, k_new, v_new, k_cache: np.ndarray, v_cache: np.ndarray, n_q_heads: int,
              n_kv_heads: int, head_dim: int, ctx_cap: int, pos: int, scale: float = 0.0):
    """k_cache / v_cache: uint16 [n_kv_heads, ctx_cap, head_dim], updated in place."""
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
    assert k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]
    assert k_cache.size == n_kv_heads * ctx_cap * head_dim
    out = np.empty(n_q_heads * head_dim, np.float64)
    _check(lib().or_attention(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                              n_q_heads, n_kv_heads, head_dim, ctx_cap, pos, scale, _ptr(out)),
           "attention")
    return out


# ---- decode step -------------------------------------------------------------------
class _Config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("ctx_cap", C.c_int64), ("rms_eps", C.c_double),
                ("rope_theta", C.c_double)]


class _Tensor(C.Structure):
    _fields_ = [("type", C.c_int), ("data", C.c_void_p)]


class _Layer(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("wq", _Tensor), ("wk", _Tensor), ("wv", _Tensor),
                ("wo", _Tensor), ("ffn_norm", C.c_void_p), ("w_gate", _Tensor),
                ("w_up", _Tensor), ("w_down", _Tensor)]


class _Model(C.Structure):
    _fields_ = [("tok_embd", _Tensor), ("output_norm", C.c_void_p), ("output", _Tensor),
                ("layers", C.POINTER(_Layer))]


@dataclass
class Config:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    ctx_cap: int
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0


@dataclass
class QTensor:
    """A packed weight matrix in host memory: `type` id and its bytes."""
    type: int
    data: np.ndarray


@dataclass
class LayerWeights:
    attn_norm: np.ndarray
    wq: QTensor
    wk: QTensor
    wv: QTensor
    wo: QTensor
    ffn_norm: np.ndarray
    w_gate: QTensor
    w_up: QTensor
    w_down: QTensor


@dataclass
class ModelWeights:
    tok_embd: QTensor
    output_norm: np.ndarray
    output: QTensor
    layers: list = field(default_factory=list)


class Decoder:
    """Holds one model plus its fp16 KV cache and runs or_decode_step."""

    def __init__(self, cfg: Config, w: ModelWeights, kv_k: np.ndarray, kv_v: np.ndarray):
        self.cfg, self.w = cfg, w
        shape = (cfg.n_layers, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim)
        assert kv_k.shape == shape and kv_v.shape == shape
        assert kv_k.dtype == np.uint16 and kv_v.dtype == np.uint16
        self.kv_k, self.kv_v = kv_k, kv_v
        self._keep = []

        def t(q: QTensor):
            d = np.ascontiguousarray(q.data, dtype=np.uint8)
            self._keep.append(d)
            return _Tensor(q.type, d.ctypes.data)

        def f(a):
            a = np.ascontiguousarray(a, dtype=np.float32)
            self._keep.append(a)
            return a.ctypes.data

        layers = (_Layer * cfg.n_layers)()
        for i, L in enumerate(w.layers):
            layers[i] = _Layer(f(L.attn_norm), t(L.wq), t(L.wk), t(L.wv), t(L.wo),
                               f(L.ffn_norm), t(L.w_gate), t(L.w_up), t(L.w_down))
        self._layers = layers
        self._model = _Model(t(w.tok_embd), f(w.output_norm), t(w.output), layers)
        self._cfg = _Config(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads,
                            cfg.head_dim, cfg.ffn, cfg.vocab, cfg.ctx_cap, cfg.rms_eps,
                            cfg.rope_theta)

    def step(self, token: int, pos: int, nthreads: int | None = None):
        """Returns (logits fp64[vocab], next token).  Updates the KV cache."""
        logits = np.empty(self.cfg.vocab, np.float64)
        nxt = C.c_int32(0)
        _check(lib().or_decode_step(C.byref(self._cfg), C.byref(self._model),
                                    _ptr(self.kv_k), _ptr(self.kv_v), int(token), int(pos),
                                    _ptr(logits), C.byref(nxt), nthreads or default_threads()),
               "decode_step")
        return logits, int(nxt.value)
