"""Synthetic Llama-shaped models built directly in device memory.

Weights are fp32 N(0, 0.02) draws from a seeded per-tensor torch generator on
the GPU, encoded by the library's own block encoder (nt_quantize) in chunks;
norm gains are 1.0; the KV cache holds N(0,1) fp16 values in the prefilled
positions.  Used by the benchmark, where generating tens of GB of weights on
the host would take minutes.  (The parity tests build their models with the
host-side generators and the oracle's encoder instead.)
"""
from __future__ import annotations

import numpy as np
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


def value_chunks(rows: int, cols: int, seed: int, stream_id: int, device, std: float = 0.02,
                 chunk_elems: int = 1 << 26):
    """Yields (first_row, n_rows, values): the seeded N(0, std) fp32 values of
    a rows x cols matrix, drawn on the device by torch's generator in row
    chunks (the same values on every call)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream_id)
    rc = max(1, chunk_elems // cols)
    for r0 in range(0, rows, rc):
        n = min(rc, rows - r0)
        w = torch.randn(n * cols, generator=g, device=device, dtype=torch.float32)
        w.mul_(std)
        yield r0, n, w


def encode_into(out: torch.Tensor, qtype: int, rows: int, cols: int, seed: int, stream_id: int,
                std: float = 0.02, chunk_elems: int = 1 << 26):
    """Fill `out` (uint8, rows x row_bytes) with encoded N(0, std) values."""
    rb = nt.row_bytes(qtype, cols)
    for r0, n, w in value_chunks(rows, cols, seed, stream_id, out.device, std, chunk_elems):
        nt.nt_quantize(qtype, w, out[r0 * rb:(r0 + n) * rb], n * cols)
        del w


def matrix_specs(s: ModelShape, streamed_from: int | None = None):
    """Every quantized matrix of the model as (layer or None, name, rows, cols,
    type, generator stream id); layers >= streamed_from are left out."""
    types = tensor_types(s.weights)
    out = [(None, "tok_embd", *matrix_shape(s, "tok_embd"), types["tok_embd"], 1),
           (None, "output", *matrix_shape(s, "output"), types["output"], 2)]
    for l in range(s.n_layers):
        if streamed_from is not None and l >= streamed_from:
            continue
        for i, name in enumerate(MATS):
            out.append((l, name, *matrix_shape(s, name), types[name], 16 + 16 * l + i))
    return out


def build(s: ModelShape, seed: int = 0, device=None, streamed_from: int | None = None):
    """Returns (Model, extras).  streamed_from: layers >= this get no device
    weights (they are served by nt_stream_layers from host blobs)."""
    dev = device or torch.device("cuda:0")
    types = tensor_types(s.weights)
    mats = {}
    for l, name, rows, cols, t, sid in matrix_specs(s, streamed_from):
        out = torch.empty(rows * nt.row_bytes(t, cols), dtype=torch.uint8, device=dev)
        encode_into(out, t, rows, cols, seed, sid)
        mats[(l, name)] = (t, out)

    ones = torch.ones(s.hidden, dtype=torch.float32, device=dev)
    layers = []
    for l in range(s.n_layers):
        lw = {"attn_norm": ones, "ffn_norm": ones}
        for name in MATS:
            lw[name] = mats.get((l, name), (types[name], None))
        layers.append(lw)
    weights = {"tok_embd": mats[(None, "tok_embd")], "output": mats[(None, "output")], "output_norm": ones,
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
    return model, dict(weights=weights, types=types, k_cache=caches[0], v_cache=caches[1])


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


def fill_streamed_blobs(s: ModelShape, first: int, seed: int = 0, device=None, last: int | None = None):
    """Pinned host blobs for layers [first, last) (last defaults to n_layers)
    in nt_layer_blob_layout order."""
    dev = device or torch.device("cuda:0")
    types = tensor_types(s.weights)
    tlist = [types[n] for n in MATS]
    cfg = nt.model_config(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                          s.ctx_cap, s.rms_eps, s.rope_theta)
    offs, nbytes = nt.nt_layer_blob_layout(cfg, tlist)
    stage = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    # one pinned region sliced per layer (a pinned allocator may round each
    # separate allocation up to a power of two)
    last = s.n_layers if last is None else last
    ns = last - first
    pinned = torch.empty(max(ns, 1) * nbytes, dtype=torch.uint8, pin_memory=True)
    blobs = []
    for l in range(first, last):
        for i, name in enumerate(MATS):
            rows, cols = matrix_shape(s, name)
            size = rows * nt.row_bytes(types[name], cols)
            encode_into(stage[offs[i]:offs[i] + size], types[name], rows, cols, seed, 16 + 16 * l + i)
        h = pinned[(l - first) * nbytes:(l - first + 1) * nbytes]
        h.copy_(stage)
        blobs.append(h)
    torch.cuda.synchronize()
    return blobs, nbytes


FILE_ALIGN = 4096


def write_layer_file(path, blobs, nbytes: int) -> int:
    """Writes layer blobs (host numpy uint8 arrays or CPU tensors of nbytes
    each) back to back at a stride of nbytes rounded up to 4096, so blob j
    starts at j * stride; returns the stride."""
    stride = (nbytes + FILE_ALIGN - 1) // FILE_ALIGN * FILE_ALIGN
    pad = bytes(stride - nbytes)
    with open(path, "wb") as fh:
        for b in blobs:
            a = b if isinstance(b, np.ndarray) else b.numpy()
            fh.write(memoryview(np.ascontiguousarray(a)))
            fh.write(pad)
    return stride


def write_streamed_file(s: ModelShape, first: int, path, seed: int = 0, device=None):
    """Layers [first, n_layers) of the device-built model as a layer file
    (nt_layer_blob_layout order, 4096-byte stride); returns (stride, blob bytes)."""
    dev = device or torch.device("cuda:0")
    types = tensor_types(s.weights)
    tlist = [types[n] for n in MATS]
    cfg = nt.model_config(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                          s.ctx_cap, s.rms_eps, s.rope_theta)
    offs, nbytes = nt.nt_layer_blob_layout(cfg, tlist)
    stage = torch.zeros(nbytes, dtype=torch.uint8, device=dev)

    def blobs():
        for l in range(first, s.n_layers):
            for i, name in enumerate(MATS):
                rows, cols = matrix_shape(s, name)
                size = rows * nt.row_bytes(types[name], cols)
                encode_into(stage[offs[i]:offs[i] + size], types[name], rows, cols, seed, 16 + 16 * l + i)
            yield stage.cpu()

    stride = write_layer_file(path, blobs(), nbytes)
    return stride, nbytes
