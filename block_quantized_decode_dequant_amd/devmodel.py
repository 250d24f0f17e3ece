"""Synthetic Llama-shaped models built directly in device memory.

Weights are fp32 N(0, 0.02) draws from a seeded per-tensor torch generator on
the GPU, encoded by the library's own block encoder (nt_quantize) in chunks;
norm gains are 1.0; the KV cache holds N(0,1) fp16 values in the prefilled
positions.  Used by the benchmark, where generating tens of GB of weights on
the host would take minutes.  (The parity tests build their models with the
host-side generators and the oracle's encoder instead.)
"""
from __future__ import annotations

import torch

from . import nt
from .workloads import ModelShape

MATS = nt.Model.MATS


def tensor_types(weights: str) -> dict:
    """Per-tensor formats: one format everywhere, or "mix" = Q4_K with Q6_K for
    attn_v, ffn_down and the output head."""
    if weights == "mix":
        return dict(tok_embd=nt.Q4_K, output=nt.Q6_K, wq=nt.Q4_K, wk=nt.Q4_K, wv=nt.Q6_K, wo=nt.Q4_K,
                    w_gate=nt.Q4_K, w_up=nt.Q4_K, w_down=nt.Q6_K)
    t = nt.QTYPES[weights]
    return {k: t for k in ("tok_embd", "output") + MATS}


def matrix_shape(s: ModelShape, name: str):
    H, QD, KD, F = s.hidden, s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim, s.ffn
    return {"tok_embd": (s.vocab, H), "output": (s.vocab, H), "wq": (QD, H), "wk": (KD, H), "wv": (KD, H),
            "wo": (H, QD), "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F)}[name]


def encode_into(out: torch.Tensor, qtype: int, rows: int, cols: int, seed: int, stream_id: int,
                std: float = 0.02, chunk_elems: int = 1 << 26):
    """Fill `out` (uint8, rows x row_bytes) with encoded N(0, std) values."""
    rb = nt.row_bytes(qtype, cols)
    g = torch.Generator(device=out.device)
    g.manual_seed(seed * 1_000_003 + stream_id)
    rc = max(1, chunk_elems // cols)
    for r0 in range(0, rows, rc):
        n = min(rc, rows - r0)
        w = torch.randn(n * cols, generator=g, device=out.device, dtype=torch.float32)
        w.mul_(std)
        nt.nt_quantize(qtype, w, out[r0 * rb:(r0 + n) * rb], n * cols)
        del w


def build(s: ModelShape, seed: int = 0, device=None, streamed_from: int | None = None):
    """Returns (Model, extras).  streamed_from: layers >= this get no device
    weights (they are served by nt_stream_layers from host blobs)."""
    dev = device or torch.device("cuda:0")
    types = tensor_types(s.weights)

    def qmat(name, sid):
        rows, cols = matrix_shape(s, name)
        t = types[name]
        out = torch.empty(rows * nt.row_bytes(t, cols), dtype=torch.uint8, device=dev)
        encode_into(out, t, rows, cols, seed, sid)
        return (t, out)

    ones = torch.ones(s.hidden, dtype=torch.float32, device=dev)
    layers = []
    for l in range(s.n_layers):
        lw = {"attn_norm": ones, "ffn_norm": ones}
        for i, name in enumerate(MATS):
            if streamed_from is not None and l >= streamed_from:
                lw[name] = (types[name], None)
            else:
                lw[name] = qmat(name, 16 + 16 * l + i)
        layers.append(lw)
    weights = {"tok_embd": qmat("tok_embd", 1), "output": qmat("output", 2), "output_norm": ones,
               "layers": layers}
    cfg = nt.model_config(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                          s.ctx_cap, s.rms_eps, s.rope_theta)
    kv_shape = (s.n_layers, s.n_kv_heads, s.ctx_cap, s.head_dim)
    g = torch.Generator(device=dev)
    g.manual_seed(seed * 1_000_003 + 999)
    caches = []
    for _ in range(2):
        c = torch.zeros(kv_shape, dtype=torch.float16, device=dev)
        c[:, :, :s.ctx, :] = torch.randn((s.n_layers, s.n_kv_heads, s.ctx, s.head_dim), generator=g,
                                         device=dev).to(torch.float16)
        caches.append(c)
    ws = torch.empty(nt.nt_model_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    model = nt.Model(cfg, weights, caches[0], caches[1], ws)
    return model, dict(weights=weights, types=types)


def weight_bytes_per_token(s: ModelShape) -> int:
    """Bytes of weights one decode step reads: every layer matrix, the output
    head and one embedding row."""
    types = tensor_types(s.weights)
    per_layer = 0
    for name in MATS:
        rows, cols = matrix_shape(s, name)
        per_layer += rows * nt.row_bytes(types[name], cols)
    head = s.vocab * nt.row_bytes(types["output"], s.hidden)
    emb_row = nt.row_bytes(types["tok_embd"], s.hidden)
    return s.n_layers * per_layer + head + emb_row


def kv_bytes_per_token(s: ModelShape, pos: int) -> int:
    """fp16 K and V read by attention at position pos (slots 0..pos), all layers."""
    return s.n_layers * 2 * s.n_kv_heads * (pos + 1) * s.head_dim * 2


def fill_streamed_blobs(s: ModelShape, first: int, seed: int = 0, device=None):
    """Pinned host blobs for layers [first, n_layers) in nt_layer_blob_layout order."""
    dev = device or torch.device("cuda:0")
    types = tensor_types(s.weights)
    tlist = [types[n] for n in MATS]
    cfg = nt.model_config(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                          s.ctx_cap, s.rms_eps, s.rope_theta)
    offs, nbytes = nt.nt_layer_blob_layout(cfg, tlist)
    stage = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    # one pinned region sliced per layer (a pinned allocator may round each
    # separate allocation up to a power of two)
    ns = s.n_layers - first
    pinned = torch.empty(max(ns, 1) * nbytes, dtype=torch.uint8, pin_memory=True)
    blobs = []
    for l in range(first, s.n_layers):
        for i, name in enumerate(MATS):
            rows, cols = matrix_shape(s, name)
            size = rows * nt.row_bytes(types[name], cols)
            encode_into(stage[offs[i]:offs[i] + size], types[name], rows, cols, seed, 16 + 16 * l + i)
        h = pinned[(l - first) * nbytes:(l - first + 1) * nbytes]
        h.copy_(stage)
        blobs.append(h)
    torch.cuda.synchronize()
    return blobs, nbytes
