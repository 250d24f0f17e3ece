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

NT_OK, NT_EINVAL, NT_ESHAPE, NT_EALIGN, NT_ENOMEM, NT_EHIP, NT_ESTATE, NT_ENODEV, NT_EIO = range(9)
F32, F16, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 0, 1, 2, 8, 12, 13, 14
QTYPES = {"f32": F32, "f16": F16, "q4_0": Q4_0, "q8_0": Q8_0, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K}
BLOCK_ELEMS = {Q8_0: 32, Q4_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 144, Q5_K: 176, Q6_K: 210}


class AttnDesc(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ctx_cap", C.c_int32), ("scale", C.c_float), ("rope_theta", C.c_float)]


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
        "nt_gemv_launch_info": (st, [i32, i64, i64, C.POINTER(C.c_int32)]),
        "nt_gemv_multi": (st, [i32, i32, C.POINTER(vp), C.POINTER(i64), C.POINTER(vp), i64, vp, vp, C.c_float,
                               i32, vp]),
        "nt_gemv_swiglu": (st, [i32, vp, vp, i64, i64, vp, vp, C.c_float, vp, vp]),
        "nt_gemm_batch_workspace_bytes": (C.c_size_t, [i32, i64, i64]),
        "nt_gemm_batch": (st, [i32, vp, vp, vp, i64, i64, i32, i32, vp, C.c_size_t, vp]),
        "nt_read_bytes": (st, [vp, i64, vp, vp]),
        "nt_copy_bytes": (st, [vp, vp, i64, vp]),
        "nt_rmsnorm": (st, [vp, vp, vp, i64, C.c_float, vp]),
        "nt_rope": (st, [vp, vp, C.c_int32, C.c_int32, C.c_int32, vp, C.c_float, vp]),
        "nt_softmax": (st, [vp, i64, vp]),
        "nt_swiglu": (st, [vp, vp, vp, i64, vp]),
        "nt_argmax": (st, [vp, i64, vp, vp]),
        "nt_embed": (st, [i32, vp, i64, i64, vp, vp, vp]),
        "nt_attn_workspace_bytes": (C.c_size_t, [C.POINTER(AttnDesc)]),
        "nt_attn_decode": (st, [C.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]),
    }
    for t in ("q8_0", "q4_0", "q4_k", "q5_k", "q6_k"):
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
def nt_dequant_q5_k(blocks, out, n, stream=None): nt_dequant(Q5_K, blocks, out, n, stream)
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
def nt_gemv_q5_k(W, x, y, rows, cols, accumulate=False, stream=None): nt_gemv(Q5_K, W, x, y, rows, cols, accumulate, stream)
def nt_gemv_q6_k(W, x, y, rows, cols, accumulate=False, stream=None): nt_gemv(Q6_K, W, x, y, rows, cols, accumulate, stream)


def nt_gemv_launch_info(qtype: int, rows: int, cols: int) -> dict:
    info = (C.c_int32 * 4)()
    _check(lib().nt_gemv_launch_info(qtype, rows, cols, info), "nt_gemv_launch_info")
    return {"fast": bool(info[0]), "vec": {2: 16, 1: 4}.get(info[0], 0), "rows_per_wg": info[1],
            "workgroups": info[2], "threads": info[3]}


def nt_gemv_multi(qtype: int, Ws, rows, ys, cols: int, x, gain=None, eps: float = 0.0,
                  accumulate: bool = False, stream=None):
    """ys[s] (+)= Ws[s] . n, n = x or RMSNorm(x, gain, eps); up to three matrices."""
    k = len(Ws)
    if not (len(rows) == k == len(ys)):
        raise ValueError("Ws, rows and ys must have the same length")
    rb = row_bytes(qtype, cols)
    W_arr = (C.c_void_p * k)(*[_ptr(W, r * rb, "W").value for W, r in zip(Ws, rows)])
    r_arr = (C.c_int64 * k)(*rows)
    y_arr = (C.c_void_p * k)(*[_ptr(y, 4 * r, "y").value for y, r in zip(ys, rows)])
    _check(lib().nt_gemv_multi(qtype, k, W_arr, r_arr, y_arr, cols, _ptr(x, 4 * cols, "x"),
                               _ptr(gain, 4 * cols, "gain"), float(eps), int(bool(accumulate)), _stream(stream)),
           "nt_gemv_multi")


def nt_gemv_swiglu(qtype: int, W_gate, W_up, rows: int, cols: int, x, h, gain=None, eps: float = 0.0,
                   stream=None):
    """h = silu(W_gate . n) * (W_up . n), n = x or RMSNorm(x, gain, eps)."""
    rb = row_bytes(qtype, cols)
    _check(lib().nt_gemv_swiglu(qtype, _ptr(W_gate, rows * rb, "W_gate"), _ptr(W_up, rows * rb, "W_up"), rows, cols,
                                _ptr(x, 4 * cols, "x"), _ptr(gain, 4 * cols, "gain"), float(eps),
                                _ptr(h, 4 * rows, "h"), _stream(stream)), "nt_gemv_swiglu")


# ---- batched verify pass -------------------------------------------------------------------
def nt_gemm_batch_workspace_bytes(qtype: int, rows: int, cols: int) -> int:
    return lib().nt_gemm_batch_workspace_bytes(qtype, rows, cols)


def nt_gemm_batch(qtype: int, W, X, Y, rows: int, cols: int, k: int, workspace, accumulate: bool = False,
                  stream=None):
    """Y[n] (+)= W . X[n] for n < k (X: k x cols, Y: k x rows, fp32, back to back).
    workspace: at least nt_gemm_batch_workspace_bytes(qtype, rows, cols) bytes
    on the device whose first 16384 bytes (the split counters) are zero
    before its first use, e.g. torch.zeros; every call leaves them zero."""
    rb = row_bytes(qtype, cols)
    need_w = rows * rb if rb > 0 else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nt_gemm_batch(qtype, _ptr(W, need_w, "W"), _ptr(X, 4 * k * cols, "X"), _ptr(Y, 4 * k * rows, "Y"),
                               rows, cols, k, int(bool(accumulate)), _ptr(workspace, 0, "workspace"), ws_bytes,
                               _stream(stream)), "nt_gemm_batch")


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


# ---- per-token ops --------------------------------------------------------------------
def nt_rmsnorm(x, gain, y, n: int, eps: float, stream=None):
    _check(lib().nt_rmsnorm(_ptr(x, 4 * n, "x"), _ptr(gain, 4 * n, "gain"), _ptr(y, 4 * n, "y"), n, eps,
                            _stream(stream)), "nt_rmsnorm")


def nt_rope(q, k, n_q_heads: int, n_kv_heads: int, head_dim: int, d_pos, theta: float, stream=None):
    _check(lib().nt_rope(_ptr(q, 4 * n_q_heads * head_dim, "q"), _ptr(k, 4 * n_kv_heads * head_dim, "k"),
                         n_q_heads, n_kv_heads, head_dim, _ptr(d_pos, 4, "d_pos"), theta, _stream(stream)),
           "nt_rope")


def nt_softmax(x, n: int, stream=None):
    _check(lib().nt_softmax(_ptr(x, 4 * n, "x"), n, _stream(stream)), "nt_softmax")


def nt_swiglu(gate, up, out, n: int, stream=None):
    _check(lib().nt_swiglu(_ptr(gate, 4 * n, "gate"), _ptr(up, 4 * n, "up"), _ptr(out, 4 * n, "out"), n,
                           _stream(stream)), "nt_swiglu")


def nt_argmax(x, n: int, out, stream=None):
    _check(lib().nt_argmax(_ptr(x, 4 * n, "x"), n, _ptr(out, 4, "out"), _stream(stream)), "nt_argmax")


def nt_embed(qtype: int, table, vocab: int, hidden: int, d_token, out, stream=None):
    rb = row_bytes(qtype, hidden)
    _check(lib().nt_embed(qtype, _ptr(table, vocab * max(rb, 0), "table"), vocab, hidden,
                          _ptr(d_token, 4, "d_token"), _ptr(out, 4 * hidden, "out"), _stream(stream)),
           "nt_embed")


def attn_desc(n_q_heads: int, n_kv_heads: int, head_dim: int, ctx_cap: int, scale: float = 0.0,
              rope_theta: float = 0.0) -> AttnDesc:
    return AttnDesc(n_q_heads, n_kv_heads, head_dim, ctx_cap, scale, rope_theta)


def nt_attn_workspace_bytes(desc: AttnDesc) -> int:
    return lib().nt_attn_workspace_bytes(C.byref(desc))


def nt_attn_decode(desc: AttnDesc, q, k_new, v_new, k_cache, v_cache, d_pos, out, workspace, stream=None):
    kv = desc.n_kv_heads * desc.head_dim
    cache = 2 * kv * desc.ctx_cap
    ws_bytes = workspace.numel() * workspace.element_size() if not isinstance(workspace, int) else 0
    _check(lib().nt_attn_decode(C.byref(desc), _ptr(q, 4 * desc.n_q_heads * desc.head_dim, "q"),
                                _ptr(k_new, 4 * kv, "k_new"), _ptr(v_new, 4 * kv, "v_new"),
                                _ptr(k_cache, cache, "k_cache"), _ptr(v_cache, cache, "v_cache"),
                                _ptr(d_pos, 4, "d_pos"), _ptr(out, 4 * desc.n_q_heads * desc.head_dim, "out"),
                                _ptr(workspace, 0, "workspace"), ws_bytes, _stream(stream)), "nt_attn_decode")


# ---- decode step and streamed layers ------------------------------------------------
class ModelConfig(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("ctx_cap", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_float)]


class TensorRef(C.Structure):
    _fields_ = [("type", C.c_int32), ("data", C.c_void_p)]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("wq", TensorRef), ("wk", TensorRef), ("wv", TensorRef),
                ("wo", TensorRef), ("ffn_norm", C.c_void_p), ("w_gate", TensorRef),
                ("w_up", TensorRef), ("w_down", TensorRef)]


class ModelWeights(C.Structure):
    _fields_ = [("tok_embd", TensorRef), ("output_norm", C.c_void_p), ("output", TensorRef),
                ("layers", C.POINTER(LayerWeights)), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t)]


class StreamDesc(C.Structure):
    _fields_ = [("first_streamed_layer", C.c_int32), ("h_layer_blobs", C.POINTER(C.c_void_p)),
                ("d_buf", C.c_void_p * 2), ("buf_bytes", C.c_size_t), ("copy_stream", C.c_void_p)]


class StreamStats(C.Structure):
    _fields_ = [("steps", C.c_uint64), ("layers_streamed", C.c_uint64), ("h2d_bytes", C.c_uint64),
                ("copy_ms", C.c_double), ("compute_ms", C.c_double), ("wall_ms", C.c_double)]


class FileTier(C.Structure):
    _fields_ = [("path", C.c_char_p), ("first_file_layer", C.c_int32), ("offset", C.c_uint64),
                ("stride", C.c_uint64), ("h_staging", C.c_void_p * 2), ("staging_bytes", C.c_size_t),
                ("direct", C.c_int32)]


class FileStats(C.Structure):
    _fields_ = [("reads", C.c_uint64), ("read_bytes", C.c_uint64), ("read_ms", C.c_double),
                ("read_span_ms", C.c_double), ("direct", C.c_int32), ("file_layers", C.c_int32)]


def _declare_model(L):
    vp, st = C.c_void_p, C.c_int
    sig = {
        "nt_model_workspace_bytes": (C.c_size_t, [C.POINTER(ModelConfig)]),
        "nt_model_create": (st, [C.POINTER(ModelConfig), C.POINTER(ModelWeights), C.POINTER(vp)]),
        "nt_model_destroy": (None, [vp]),
        "nt_model_set_graph": (st, [vp, C.c_int]),
        "nt_decode_step": (st, [vp, vp, vp, vp, vp, vp]),
        "nt_layer_blob_layout": (st, [C.POINTER(ModelConfig), C.POINTER(C.c_int32), C.POINTER(C.c_size_t),
                                      C.POINTER(C.c_size_t)]),
        "nt_stream_layers": (st, [vp, C.POINTER(StreamDesc)]),
        "nt_stream_stats_get": (st, [vp, C.POINTER(StreamStats)]),
        "nt_stream_layers_tiered": (st, [vp, C.POINTER(StreamDesc), C.POINTER(FileTier)]),
        "nt_file_stats_get": (st, [vp, C.POINTER(FileStats)]),
        "nt_tier_plan": (st, [C.POINTER(ModelConfig), C.POINTER(C.c_int32), C.c_uint64, C.c_uint64,
                              C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def model_config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, ctx_cap,
                 rms_eps=1e-5, rope_theta=500000.0) -> ModelConfig:
    return ModelConfig(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, ctx_cap,
                       rms_eps, rope_theta)


def nt_model_workspace_bytes(cfg: ModelConfig) -> int:
    _declare_model(lib())
    return lib().nt_model_workspace_bytes(C.byref(cfg))


def nt_tier_plan(cfg: ModelConfig, types, vram_bytes: int, pinned_bytes: int):
    """(first_streamed_layer, first_file_layer) for the given tier capacities."""
    _declare_model(lib())
    t = (C.c_int32 * 7)(*types)
    a, b = C.c_int32(0), C.c_int32(0)
    _check(lib().nt_tier_plan(C.byref(cfg), t, int(vram_bytes), int(pinned_bytes), C.byref(a), C.byref(b)),
           "nt_tier_plan")
    return int(a.value), int(b.value)


def nt_layer_blob_layout(cfg: ModelConfig, types):
    _declare_model(lib())
    t = (C.c_int32 * 7)(*types)
    offs = (C.c_size_t * 7)()
    nb = C.c_size_t(0)
    _check(lib().nt_layer_blob_layout(C.byref(cfg), t, offs, C.byref(nb)), "nt_layer_blob_layout")
    return list(offs), int(nb.value)


class Model:
    """Owns an nt_model handle; keeps the tensors it points at alive.

    weights: dict with tok_embd, output (each (qtype, uint8 tensor)), output_norm
    (fp32 tensor) and layers: list of dicts with attn_norm, ffn_norm (fp32) and
    wq, wk, wv, wo, w_gate, w_up, w_down ((qtype, uint8 tensor) or (qtype, None)).
    """

    MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")

    def __init__(self, cfg: ModelConfig, weights: dict, k_cache, v_cache, workspace):
        L = lib()
        _declare_model(L)
        self.cfg = cfg
        self._keep = [weights, k_cache, v_cache, workspace]

        def ref(pair):
            t, tensor = pair
            return TensorRef(t, None if tensor is None else _ptr(tensor, 0, "weight").value)

        layers = (LayerWeights * cfg.n_layers)()
        for i, lw in enumerate(weights["layers"]):
            layers[i] = LayerWeights(_ptr(lw["attn_norm"], 4 * cfg.hidden).value, ref(lw["wq"]), ref(lw["wk"]),
                                     ref(lw["wv"]), ref(lw["wo"]), _ptr(lw["ffn_norm"], 4 * cfg.hidden).value,
                                     ref(lw["w_gate"]), ref(lw["w_up"]), ref(lw["w_down"]))
        self._layers = layers
        kv = 2 * cfg.n_layers * cfg.n_kv_heads * cfg.ctx_cap * cfg.head_dim
        ws_bytes = workspace.numel() * workspace.element_size()
        w = ModelWeights(ref(weights["tok_embd"]), _ptr(weights["output_norm"], 4 * cfg.hidden).value,
                         ref(weights["output"]), layers, _ptr(k_cache, kv, "k_cache").value,
                         _ptr(v_cache, kv, "v_cache").value, _ptr(workspace, 0, "workspace").value, ws_bytes)
        h = C.c_void_p()
        _check(L.nt_model_create(C.byref(cfg), C.byref(w), C.byref(h)), "nt_model_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) and self.handle.value:
            lib().nt_model_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_graph(self, enable: bool):
        _check(lib().nt_model_set_graph(self.handle, int(bool(enable))), "nt_model_set_graph")

    def step(self, d_token, d_pos, logits, d_next, stream=None):
        _check(lib().nt_decode_step(self.handle, _ptr(d_token, 4, "d_token"), _ptr(d_pos, 4, "d_pos"),
                                    _ptr(logits, 4 * self.cfg.vocab, "logits"), _ptr(d_next, 4, "d_next"),
                                    _stream(stream)), "nt_decode_step")

    def stream_layers(self, first_streamed: int, host_blobs, d_buf0, d_buf1, copy_stream):
        """host_blobs: list of pinned host uint8 tensors (one per streamed layer)."""
        if host_blobs is None:
            _check(lib().nt_stream_layers(self.handle, None), "nt_stream_layers")
            return
        n = len(host_blobs)
        arr = (C.c_void_p * max(n, 1))(*[b.data_ptr() for b in host_blobs])
        self._stream_keep = [host_blobs, d_buf0, d_buf1, arr, copy_stream]
        bufs = (C.c_void_p * 2)(d_buf0.data_ptr(), d_buf1.data_ptr())
        nbytes = min(d_buf0.numel(), d_buf1.numel()) * d_buf0.element_size()
        desc = StreamDesc(first_streamed, C.cast(arr, C.POINTER(C.c_void_p)), bufs, nbytes,
                          _stream(copy_stream))
        _check(lib().nt_stream_layers(self.handle, C.byref(desc)), "nt_stream_layers")

    def stream_layers_tiered(self, first_streamed: int, host_blobs, d_buf0, d_buf1, copy_stream, path: str,
                             first_file: int, offset: int, stride: int, staging0, staging1, direct: bool = True):
        """As stream_layers, with layers [first_file, n_layers) read from `path`
        (blob j at offset + j * stride) through the pinned host staging
        tensors staging0 / staging1; host_blobs covers [first_streamed, first_file)."""
        n = len(host_blobs)
        arr = (C.c_void_p * max(n, 1))(*[b.data_ptr() for b in host_blobs])
        bufs = (C.c_void_p * 2)(d_buf0.data_ptr(), d_buf1.data_ptr())
        nbytes = min(d_buf0.numel(), d_buf1.numel()) * d_buf0.element_size()
        desc = StreamDesc(first_streamed, C.cast(arr, C.POINTER(C.c_void_p)), bufs, nbytes, _stream(copy_stream))
        sbytes = min(staging0.numel(), staging1.numel()) * staging0.element_size()
        pbytes = path.encode()
        ft = FileTier(pbytes, first_file, offset, stride, (C.c_void_p * 2)(staging0.data_ptr(), staging1.data_ptr()),
                      sbytes, int(bool(direct)))
        self._stream_keep = [host_blobs, d_buf0, d_buf1, arr, copy_stream, staging0, staging1, pbytes]
        _check(lib().nt_stream_layers_tiered(self.handle, C.byref(desc), C.byref(ft)), "nt_stream_layers_tiered")

    def file_stats(self) -> dict:
        s = FileStats()
        _check(lib().nt_file_stats_get(self.handle, C.byref(s)), "nt_file_stats_get")
        return {k: getattr(s, k) for k, _ in FileStats._fields_}

    def stream_stats(self) -> dict:
        s = StreamStats()
        _check(lib().nt_stream_stats_get(self.handle, C.byref(s)), "nt_stream_stats_get")
        return {k: getattr(s, k) for k, _ in StreamStats._fields_}


# ---- GGUF model files (host-side reader in libnt) -------------------------------------
def _declare_gguf(L):
    vp, st, i64 = C.c_void_p, C.c_int, C.c_int64
    sig = {
        "nt_gguf_open": (st, [C.c_char_p, C.POINTER(vp)]),
        "nt_gguf_close": (None, [vp]),
        "nt_gguf_tensor_count": (i64, [vp]),
        "nt_gguf_find_tensor": (i64, [vp, C.c_char_p]),
        "nt_gguf_tensor_info": (st, [vp, i64, C.POINTER(C.c_char_p), C.POINTER(C.c_int32), C.POINTER(i64),
                                     C.POINTER(i64), C.POINTER(vp), C.POINTER(C.c_size_t)]),
        "nt_gguf_llama_config": (st, [vp, C.c_int32, C.POINTER(ModelConfig)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


class GGUF:
    """An open GGUF file (libnt maps it read-only).  tensor(name) returns
    (type, rows, cols, read-only numpy uint8 view of the mapped bytes); the
    views are valid until close()."""

    def __init__(self, path: str):
        L = lib()
        _declare_gguf(L)
        h = C.c_void_p()
        _check(L.nt_gguf_open(os.fsencode(path), C.byref(h)), "nt_gguf_open")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) and self.handle.value:
            lib().nt_gguf_close(self.handle)
            self.handle = C.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __len__(self):
        return int(lib().nt_gguf_tensor_count(self.handle))

    def info(self, i: int):
        import numpy as np
        name, t, rows, cols = C.c_char_p(), C.c_int32(), C.c_int64(), C.c_int64()
        data, nbytes = C.c_void_p(), C.c_size_t()
        _check(lib().nt_gguf_tensor_info(self.handle, i, C.byref(name), C.byref(t), C.byref(rows), C.byref(cols),
                                         C.byref(data), C.byref(nbytes)), "nt_gguf_tensor_info")
        view = np.ctypeslib.as_array((C.c_uint8 * nbytes.value).from_address(data.value))
        view.flags.writeable = False
        return name.value.decode(), t.value, rows.value, cols.value, view

    def names(self):
        return [self.info(i)[0] for i in range(len(self))]

    def tensor(self, name: str):
        i = lib().nt_gguf_find_tensor(self.handle, name.encode())
        if i < 0:
            raise KeyError(name)
        _, t, rows, cols, view = self.info(i)
        return t, rows, cols, view

    def llama_config(self, ctx_cap: int = 0) -> ModelConfig:
        cfg = ModelConfig()
        _check(lib().nt_gguf_llama_config(self.handle, ctx_cap, C.byref(cfg)), "nt_gguf_llama_config")
        return cfg
