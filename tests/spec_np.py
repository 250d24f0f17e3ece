"""A second, independent reading of one batch-1 Llama decode step, in numpy
fp64, used only to pin the oracle's C decode step (test infrastructure).

It shares no code with the oracle: the block decoders, the norms, RoPE, the
fp16 KV cache, attention, SwiGLU and the greedy pick are written out again
here from the readings of the ntransformer write-up (GeekNews topic 26894):
"Main features" lists the Llama block (RoPE, GQA, SwiGLU, RMSNorm, KV cache),
"Roadmap" the F16 KV cache, "Overview" the GGUF block formats.  Readings where
the pages are silent (the same ones the oracle takes): pre-norm residual
blocks, eps inside the root, RoPE on adjacent pairs with angle
pos * theta^(-2i/D), k and v rounded to fp16 (round to nearest even) when
stored at slot pos and attended from their stored values, contiguous GQA
groups, scale 1/sqrt(D), greedy argmax with the lowest index on ties.

Only the block formats with a plain closed form are decoded here (Q8_0,
Q4_0, Q6_K); that is enough to drive every step of the block.
"""
from __future__ import annotations

import numpy as np


# ---- block decoders ("Overview": GGUF block formats) -------------------------
def _f16(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """fp16 values from little-endian byte pairs (numpy's IEEE binary16)."""
    bits = lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)
    return bits.view(np.float16).astype(np.float64)


def decode_q8_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """34-byte blocks: fp16 d, then 32 int8 codes; value = d * q."""
    b = raw[: rows * cols // 32 * 34].reshape(-1, 34)
    d = _f16(b[:, 0], b[:, 1])
    q = b[:, 2:].view(np.int8).astype(np.float64)
    return (d[:, None] * q).reshape(rows, cols)


def decode_q4_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """18-byte blocks: fp16 d, 16 bytes; byte i holds value i in its low
    nibble and value i + 16 in its high nibble; value = d * (q - 8)."""
    b = raw[: rows * cols // 32 * 18].reshape(-1, 18)
    d = _f16(b[:, 0], b[:, 1])
    qs = b[:, 2:]
    q = np.concatenate([qs & 15, qs >> 4], axis=1).astype(np.float64) - 8.0
    return (d[:, None] * q).reshape(rows, cols)


def decode_q6_k(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """210-byte super-blocks of 256: ql[128], qh[64], int8 scales[16], fp16 d.
    Value e: half h = e // 128, r = e % 128, k = r // 32, l = r % 32; the low
    four bits come from ql[64h + 32(k & 1) + l] (low nibble for k < 2, high
    otherwise), the top two from (qh[32h + l] >> 2k) & 3; value =
    d * scales[e // 16] * (q - 32)."""
    b = raw[: rows * cols // 256 * 210].reshape(-1, 210)
    ql, qh = b[:, :128].astype(np.int64), b[:, 128:192].astype(np.int64)
    sc = b[:, 192:208].view(np.int8).astype(np.float64)
    d = _f16(b[:, 208], b[:, 209])
    e = np.arange(256)
    h, r = e // 128, e % 128
    k, l = r // 32, r % 32
    lo_byte = ql[:, 64 * h + 32 * (k & 1) + l]
    lo = np.where(k < 2, lo_byte & 15, lo_byte >> 4)
    hi = (qh[:, 32 * h + l] >> (2 * k)) & 3
    q = (lo | (hi << 4)).astype(np.float64) - 32.0
    return (d[:, None] * sc[:, e // 16] * q).reshape(rows, cols)


DECODERS = {8: decode_q8_0, 2: decode_q4_0, 14: decode_q6_k}


def matrix(t: int, raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    return DECODERS[t](np.ascontiguousarray(raw, dtype=np.uint8), rows, cols)


# ---- the Llama block ("Main features") ----------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    return g * x / np.sqrt(np.mean(x * x) + eps)


def rope(v: np.ndarray, n_heads: int, d: int, pos: int, theta: float) -> np.ndarray:
    """Adjacent pairs (2i, 2i + 1) of each head turned by pos * theta^(-2i/d)."""
    x = v.reshape(n_heads, d // 2, 2)
    phi = pos * theta ** (-2.0 * np.arange(d // 2) / d)
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[:, :, 0], x[:, :, 1]
    return np.stack([a * c - b * s, a * s + b * c], axis=-1).reshape(-1)


def to_f16(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp16 (round to nearest even), as stored in the KV cache."""
    return v.astype(np.float16)


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


class SpecModel:
    """cfg: dict with n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn,
    vocab, ctx_cap, rms_eps, rope_theta.  weights: dict with tok_embd and
    output as (type, bytes), output_norm, and layers: a list of dicts with
    attn_norm, ffn_norm and wq, wk, wv, wo, w_gate, w_up, w_down as
    (type, bytes).  k_cache, v_cache: fp16 [layers, kv_heads, ctx_cap, D]."""

    def __init__(self, cfg: dict, weights: dict, k_cache: np.ndarray, v_cache: np.ndarray):
        self.c = cfg
        H, D = cfg["hidden"], cfg["head_dim"]
        QD, KD, F, V = cfg["n_q_heads"] * D, cfg["n_kv_heads"] * D, cfg["ffn"], cfg["vocab"]
        shapes = {"wq": (QD, H), "wk": (KD, H), "wv": (KD, H), "wo": (H, QD), "w_gate": (F, H),
                  "w_up": (F, H), "w_down": (H, F)}
        self.emb = matrix(*weights["tok_embd"], V, H)
        self.out = matrix(*weights["output"], V, H)
        self.out_norm = np.asarray(weights["output_norm"], np.float64)
        self.layers = []
        for L in weights["layers"]:
            m = {k: matrix(*L[k], *shapes[k]) for k in shapes}
            m["attn_norm"] = np.asarray(L["attn_norm"], np.float64)
            m["ffn_norm"] = np.asarray(L["ffn_norm"], np.float64)
            self.layers.append(m)
        self.k = k_cache.copy()
        self.v = v_cache.copy()

    def attend(self, l: int, q: np.ndarray, pos: int) -> np.ndarray:
        c = self.c
        D, hq, hk = c["head_dim"], c["n_q_heads"], c["n_kv_heads"]
        grp = hq // hk
        out = np.empty(hq * D)
        for h in range(hq):
            g = h // grp
            K = self.k[l, g, : pos + 1].astype(np.float64)
            Vv = self.v[l, g, : pos + 1].astype(np.float64)
            s = K @ q[h * D:(h + 1) * D] / np.sqrt(D)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[h * D:(h + 1) * D] = p @ Vv
        return out

    def step(self, token: int, pos: int):
        """Returns (logits fp64[vocab], greedy next token); stores k, v at pos."""
        c = self.c
        D, eps, th = c["head_dim"], c["rms_eps"], c["rope_theta"]
        hq, hk = c["n_q_heads"], c["n_kv_heads"]
        x = self.emb[token].copy()
        for l, L in enumerate(self.layers):
            n = rmsnorm(x, L["attn_norm"], eps)
            q = rope(L["wq"] @ n, hq, D, pos, th)
            k = rope(L["wk"] @ n, hk, D, pos, th)
            v = L["wv"] @ n
            self.k[l, :, pos, :] = to_f16(k).reshape(hk, D)
            self.v[l, :, pos, :] = to_f16(v).reshape(hk, D)
            x = x + L["wo"] @ self.attend(l, q, pos)
            m = rmsnorm(x, L["ffn_norm"], eps)
            x = x + L["w_down"] @ (silu(L["w_gate"] @ m) * (L["w_up"] @ m))
        logits = self.out @ rmsnorm(x, self.out_norm, eps)
        return logits, int(np.argmax(logits))   # argmax: first (lowest) index of the maximum
