"""Synthetic Llama-shaped models for the tests: seeded fp32 weights from the
shared generators, quantized by the oracle's encoders into host bytes.

Test infrastructure: it calls the oracle, so only tests use it.
"""
from __future__ import annotations

import numpy as np

import oracle as O
from block_quantized_decode_dequant_amd import synth


def tiny_config(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                vocab=1000, ctx_cap=32, rms_eps=1e-5, rope_theta=500000.0) -> O.Config:
    return O.Config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, ctx_cap,
                    rms_eps, rope_theta)


def _types(wtype):
    """Per-tensor types: one type everywhere, the mixed K-quant recipe
    (Q6_K for attn_v, ffn_down and the output head, Q4_K elsewhere), or a
    dict naming each tensor's type (keys tok, wq, wk, wv, wo, gate, up, down,
    out)."""
    if isinstance(wtype, dict):
        return dict(wtype)
    if wtype == "mix":
        base = O.Q4_K
        return dict(tok=base, wq=base, wk=base, wv=O.Q6_K, wo=base, gate=base, up=base,
                    down=O.Q6_K, out=O.Q6_K)
    return dict(tok=wtype, wq=wtype, wk=wtype, wv=wtype, wo=wtype, gate=wtype, up=wtype,
                down=wtype, out=wtype)


def _qt(t, seed, stream, rows, cols, std=0.02):
    return O.QTensor(t, O.quantize(t, synth.normal_f32(seed, stream, rows * cols, std=std)))


def build_oracle_model(cfg: O.Config, seed: int = 0, wtype=O.Q8_0, gains: str = "random"):
    """gains: "random" -> N(1, 0.1) (unit tests), "one" -> 1.0 (model workloads)."""
    ty = _types(wtype)
    H, D = cfg.hidden, cfg.head_dim
    QD, KD, F, V = cfg.n_q_heads * D, cfg.n_kv_heads * D, cfg.ffn, cfg.vocab

    def gain(stream):
        if gains == "one":
            return np.ones(H, np.float32)
        return synth.normal_f32(seed, stream, H, mean=1.0, std=0.1)

    layers = []
    for l in range(cfg.n_layers):
        s = lambda which: synth.layer_stream(l, which)
        layers.append(O.LayerWeights(
            attn_norm=gain(s(synth.ATTN_NORM)),
            wq=_qt(ty["wq"], seed, s(synth.WQ), QD, H),
            wk=_qt(ty["wk"], seed, s(synth.WK), KD, H),
            wv=_qt(ty["wv"], seed, s(synth.WV), KD, H),
            wo=_qt(ty["wo"], seed, s(synth.WO), H, QD),
            ffn_norm=gain(s(synth.FFN_NORM)),
            w_gate=_qt(ty["gate"], seed, s(synth.W_GATE), F, H),
            w_up=_qt(ty["up"], seed, s(synth.W_UP), F, H),
            w_down=_qt(ty["down"], seed, s(synth.W_DOWN), H, F)))
    return O.ModelWeights(
        tok_embd=_qt(ty["tok"], seed, synth.TOK_EMBD, V, H),
        output_norm=gain(synth.OUTPUT_NORM),
        output=_qt(ty["out"], seed, synth.OUTPUT, V, H),
        layers=layers)


def kv_prefix(cfg: O.Config, seed: int, n_pos: int):
    kk = np.stack([synth.kv_prefix_bits(seed, l, 0, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    vv = np.stack([synth.kv_prefix_bits(seed, l, 1, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    return kk, vv
