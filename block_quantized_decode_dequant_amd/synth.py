"""Seeded synthetic inputs shared by the tests, the oracle runs and the benchmark.

This module only draws numbers and lays out bytes; it holds none of the
decode arithmetic (no decoding, quantizing, norms, products).  Every stream
is a counter-based Philox4x32-10 generator (Salmon et al., SC'11, "Parallel
random numbers: as easy as 1, 2, 3") keyed by (seed, stream id), so each
tensor can be regenerated on its own, in any order, with identical values.

Recipes (the write-up measured real Llama 3.1 8B / 70B GGUF models, which are
not available here; these seeded stand-ins take their shapes):

* Q8_0 GEMV test matrix: int8 codes uniform on [-127, 127], one fp16 scale per
  32-value block equal to |N(0,1)| * 0.01 rounded to fp16, x ~ N(0,1).
* K-quant GEMV matrices and model weights: fp32 N(0, 0.02) values (quantized
  afterwards by the caller), activations x ~ N(0,1).
* KV-cache prefix: fp16 N(0,1) values in every layer's K and V.
* Norm gains: 1.0 in the model workloads; N(1, 0.1) in unit tests.
"""
from __future__ import annotations

import numpy as np

_CHUNK = 1 << 22

# Stream ids of the fixed workloads.
Q8_CFG_CODES, Q8_CFG_SCALES, Q8_CFG_X = 1, 2, 3


def rng(seed: int, stream: int) -> np.random.Generator:
    key = np.array([seed & (2**64 - 1), stream & (2**64 - 1)], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def normal_f32(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """n float32 draws of N(mean, std^2), drawn in fixed-size chunks."""
    g = rng(seed, stream)
    out = np.empty(n, np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        z = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            z *= np.float32(std)
        if mean != 0.0:
            z += np.float32(mean)
        out[lo:hi] = z
    return out


def normal_f16_bits(seed: int, stream: int, n: int) -> np.ndarray:
    """n fp16 N(0,1) draws, returned as their uint16 bit patterns."""
    return normal_f32(seed, stream, n).astype(np.float16).view(np.uint16)


def uniform_int(seed: int, stream: int, n: int, lo: int, hi: int, dtype=np.int64) -> np.ndarray:
    """n integers uniform on [lo, hi] (both ends included)."""
    return rng(seed, stream).integers(lo, hi + 1, size=n, dtype=np.int64).astype(dtype)


Q8_0_DTYPE = np.dtype([("d", "<u2"), ("qs", "i1", (32,))])


def q8_0_bytes(d_bits: np.ndarray, qs: np.ndarray) -> np.ndarray:
    """Lay out Q8_0 blocks (fp16 scale bits, then 32 int8 codes) as bytes."""
    nb = d_bits.size
    rec = np.empty(nb, Q8_0_DTYPE)
    rec["d"] = d_bits.reshape(nb)
    rec["qs"] = qs.reshape(nb, 32)
    return rec.view(np.uint8).reshape(-1)


def q8_0_random_parts(seed: int, rows: int, cols: int):
    """The Q8_0 GEMV test matrix as parts: (scale bits uint16[nblocks], codes int8[n])."""
    assert cols % 32 == 0
    n = rows * cols
    qs = uniform_int(seed, Q8_CFG_CODES, n, -127, 127, np.int8)
    z = np.abs(normal_f32(seed, Q8_CFG_SCALES, n // 32).astype(np.float64)) * 0.01
    d_bits = z.astype(np.float16).view(np.uint16)
    return d_bits, qs


def q8_0_random_matrix(seed: int, rows: int, cols: int) -> np.ndarray:
    d_bits, qs = q8_0_random_parts(seed, rows, cols)
    return q8_0_bytes(d_bits, qs)


def activation(seed: int, stream: int, n: int) -> np.ndarray:
    return normal_f32(seed, stream, n)


# ---- model tensors ----------------------------------------------------------------
# Stream id of each tensor of a synthetic Llama model.
TOK_EMBD, OUTPUT, OUTPUT_NORM = 1, 2, 3
LAYER_BASE, LAYER_STRIDE = 16, 16
ATTN_NORM, WQ, WK, WV, WO, FFN_NORM, W_GATE, W_UP, W_DOWN = range(9)
KV_BASE = 1 << 40


def layer_stream(layer: int, which: int) -> int:
    return LAYER_BASE + LAYER_STRIDE * layer + which


def kv_prefix_bits(seed: int, layer: int, which: int, n_kv_heads: int, ctx_cap: int,
                   head_dim: int, n_pos: int) -> np.ndarray:
    """fp16 bits [n_kv_heads, ctx_cap, head_dim]: N(0,1) in slots [0, n_pos), zero after."""
    out = np.zeros((n_kv_heads, ctx_cap, head_dim), np.uint16)
    if n_pos > 0:
        vals = normal_f16_bits(seed, KV_BASE + 2 * layer + which, n_kv_heads * n_pos * head_dim)
        out[:, :n_pos, :] = vals.reshape(n_kv_heads, n_pos, head_dim)
    return out
