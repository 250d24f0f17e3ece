"""Llama decode models from GGUF files: the tensors of a file opened by libnt's
GGUF reader (nt.GGUF) copied into device memory in the layout nt.Model takes.

The engine the ntransformer write-up describes loads GGUF models ("Overview");
this is the same entry point for this library.  The quantized matrices keep
their packed bytes (the block layouts are the GGUF ones), the norm gains are
F32 (F16 is widened).  A file without output.weight shares token_embd.weight
as the output head.
"""
from __future__ import annotations

import numpy as np

from . import nt

LAYER_TENSORS = {  # nt.Model name -> GGUF tensor name in block i
    "attn_norm": "attn_norm", "wq": "attn_q", "wk": "attn_k", "wv": "attn_v", "wo": "attn_output",
    "ffn_norm": "ffn_norm", "w_gate": "ffn_gate", "w_up": "ffn_up", "w_down": "ffn_down",
}


def _shapes(cfg):
    H, D, F = cfg.hidden, cfg.head_dim, cfg.ffn
    QD, KD = cfg.n_q_heads * D, cfg.n_kv_heads * D
    return {"wq": (QD, H), "wk": (KD, H), "wv": (KD, H), "wo": (H, QD), "w_gate": (F, H), "w_up": (F, H),
            "w_down": (H, F)}


def load_llama(path: str, ctx_cap: int = 0, device=None):
    """Returns (nt.ModelConfig, weights dict for nt.Model) with every tensor on
    `device` (default cuda:0).  Raises ValueError for a tensor of the wrong
    type or shape."""
    import torch

    dev = torch.device(device or "cuda:0")
    with nt.GGUF(path) as g:
        cfg = g.llama_config(ctx_cap)

        def matrix(name, rows, cols):
            t, r, c, view = g.tensor(name)
            if t not in nt.BLOCK_BYTES:
                raise ValueError(f"{name}: type {t} is not a quantized format this library decodes")
            if (r, c) != (rows, cols):
                raise ValueError(f"{name}: {r} x {c}, expected {rows} x {cols}")
            return (t, torch.from_numpy(view.copy()).to(dev))

        def gain(name):
            t, r, c, view = g.tensor(name)
            if r != 1 or c != cfg.hidden:
                raise ValueError(f"{name}: {r} x {c}, expected a vector of {cfg.hidden}")
            if t == nt.F32:
                v = view.view(np.float32)
            elif t == nt.F16:
                v = view.view(np.float16).astype(np.float32)
            else:
                raise ValueError(f"{name}: norm gains must be F32 or F16, not type {t}")
            return torch.from_numpy(v.copy()).to(dev)

        shapes = _shapes(cfg)
        layers = []
        for i in range(cfg.n_layers):
            lw = {}
            for key, gname in LAYER_TENSORS.items():
                name = f"blk.{i}.{gname}.weight"
                lw[key] = gain(name) if key.endswith("norm") else matrix(name, *shapes[key])
            layers.append(lw)
        names = set(g.names())
        head = "output.weight" if "output.weight" in names else "token_embd.weight"
        weights = {"tok_embd": matrix("token_embd.weight", cfg.vocab, cfg.hidden),
                   "output_norm": gain("output_norm.weight"),
                   "output": matrix(head, cfg.vocab, cfg.hidden),
                   "layers": layers}
    return cfg, weights
