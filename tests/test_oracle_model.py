"""Pins for the oracle's whole decode step (the Llama block of the ntransformer
write-up, GeekNews topic 26894, "Main features"; engine and sampler under
"Architecture").

Special cases make the step collapse onto primitives that are pinned on their
own: with every layer matrix zero the residual stream keeps the embedding row;
with zero query weights attention averages the cached values; with zero
attention weights only the feed-forward block moves x.
"""
import math

import numpy as np
import pytest

import oracle as O
from block_quantized_decode_dequant_amd import synth

from .model_util import build_oracle_model, tiny_config


def _zero(t, rows, cols):
    return O.QTensor(t, np.zeros(rows * O.row_bytes(t, cols), np.uint8))


def _decoder(cfg, w, seed=0, n_pos=0):
    kk = np.stack([synth.kv_prefix_bits(seed, l, 0, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    vv = np.stack([synth.kv_prefix_bits(seed, l, 1, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    return O.Decoder(cfg, w, kk, vv)


def _emb_row(w, cfg, token):
    rb = O.row_bytes(w.tok_embd.type, cfg.hidden)
    return O.dequant(w.tok_embd.type, w.tok_embd.data[token * rb:(token + 1) * rb], cfg.hidden)


def _head(w, cfg, x):
    n = O.rmsnorm(x, w.output_norm, cfg.rms_eps)
    return O.gemv(w.output.type, w.output.data, cfg.vocab, cfg.hidden, n)


def _zero_layers(cfg, w, keep=()):
    H, QD, KD, F = cfg.hidden, cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.ffn
    shapes = {"wq": (QD, H), "wk": (KD, H), "wv": (KD, H), "wo": (H, QD), "w_gate": (F, H),
              "w_up": (F, H), "w_down": (H, F)}
    for L in w.layers:
        for name, (r, c) in shapes.items():
            if name not in keep:
                setattr(L, name, _zero(getattr(L, name).type, r, c))


@pytest.mark.parametrize("wtype", [O.Q8_0, O.Q4_K])
def test_zero_layers_leave_the_embedding(wtype):
    cfg = tiny_config()
    w = build_oracle_model(cfg, seed=2, wtype=wtype)
    _zero_layers(cfg, w)
    dec = _decoder(cfg, w, n_pos=3)
    token, pos = 7, 3
    logits, nxt = dec.step(token, pos)
    ref = _head(w, cfg, _emb_row(w, cfg, token).astype(np.float64))
    assert np.allclose(logits, ref, rtol=1e-13, atol=1e-13)
    assert nxt == int(np.argmax(ref))
    # k = v = 0 were stored (rotating a zero pair may give -0.0, still zero)
    assert np.all(dec.kv_k[:, :, pos, :].view(np.float16) == 0)
    assert np.all(dec.kv_v[:, :, pos, :].view(np.float16) == 0)


def test_zero_queries_average_cached_values():
    """Wq = 0 gives equal scores, so attention is the mean of V over [0, pos]."""
    cfg = tiny_config(n_layers=1)
    w = build_oracle_model(cfg, seed=3, wtype=O.Q8_0)
    _zero_layers(cfg, w, keep=("wk", "wv", "wo"))
    dec = _decoder(cfg, w, seed=3, n_pos=5)
    token, pos = 11, 5
    x0 = _emb_row(w, cfg, token).astype(np.float64)
    n = O.rmsnorm(x0, w.layers[0].attn_norm, cfg.rms_eps)
    KD = cfg.n_kv_heads * cfg.head_dim
    k = O.gemv(w.layers[0].wk.type, w.layers[0].wk.data, KD, cfg.hidden, n)
    v = O.gemv(w.layers[0].wv.type, w.layers[0].wv.data, KD, cfg.hidden, n)
    k = O.rope(k, cfg.n_kv_heads, cfg.head_dim, pos, cfg.rope_theta)
    v_before = dec.kv_v[0].view(np.float16).astype(np.float64).copy()
    logits, _ = dec.step(token, pos)
    # the new k, v sit at slot pos, rounded to fp16
    assert np.array_equal(dec.kv_k[0, :, pos, :].reshape(-1), k.astype(np.float16).view(np.uint16))
    assert np.array_equal(dec.kv_v[0, :, pos, :].reshape(-1), v.astype(np.float16).view(np.uint16))
    vals = v_before
    vals[:, pos, :] = v.astype(np.float16).astype(np.float64).reshape(cfg.n_kv_heads, cfg.head_dim)
    grp = cfg.n_q_heads // cfg.n_kv_heads
    o = np.concatenate([vals[h // grp, : pos + 1].mean(axis=0) for h in range(cfg.n_q_heads)])
    x1 = x0 + O.gemv(w.layers[0].wo.type, w.layers[0].wo.data, cfg.hidden,
                     cfg.n_q_heads * cfg.head_dim, o)
    assert np.allclose(logits, _head(w, cfg, x1), rtol=1e-10, atol=1e-12)


def test_feed_forward_only():
    cfg = tiny_config(n_layers=1)
    w = build_oracle_model(cfg, seed=4, wtype=O.Q6_K)
    _zero_layers(cfg, w, keep=("w_gate", "w_up", "w_down"))
    dec = _decoder(cfg, w, seed=4, n_pos=2)
    token, pos = 3, 2
    x0 = _emb_row(w, cfg, token).astype(np.float64)
    L = w.layers[0]
    m = O.rmsnorm(x0, L.ffn_norm, cfg.rms_eps)
    g = O.gemv(L.w_gate.type, L.w_gate.data, cfg.ffn, cfg.hidden, m)
    u = O.gemv(L.w_up.type, L.w_up.data, cfg.ffn, cfg.hidden, m)
    x1 = x0 + O.gemv(L.w_down.type, L.w_down.data, cfg.hidden, cfg.ffn, O.swiglu(g, u))
    logits, _ = dec.step(token, pos)
    assert np.allclose(logits, _head(w, cfg, x1), rtol=1e-11, atol=1e-12)


def test_step_is_deterministic_and_uses_previous_kv():
    cfg = tiny_config()
    w = build_oracle_model(cfg, seed=5, wtype=O.Q4_K)
    a = _decoder(cfg, w, seed=5, n_pos=4)
    b = _decoder(cfg, w, seed=5, n_pos=4)
    la, ta = a.step(9, 4, nthreads=1)
    lb, tb = b.step(9, 4, nthreads=5)
    assert np.array_equal(la, lb) and ta == tb
    # the next step reads the slot the first one wrote: perturbing it changes logits
    l2, _ = a.step(ta, 5)
    b.kv_v[0, :, 4, :] = 0
    l3, _ = b.step(tb, 5)
    assert not np.array_equal(l2, l3)


def test_step_rejects_out_of_range():
    cfg = tiny_config()
    w = build_oracle_model(cfg, seed=6, wtype=O.Q8_0)
    dec = _decoder(cfg, w)
    with pytest.raises(ValueError):
        dec.step(cfg.vocab, 0)
    with pytest.raises(ValueError):
        dec.step(0, cfg.ctx_cap)


# A decode step read a second time, in numpy fp64 (tests/spec_np.py), on a
# model whose every matrix, gain and cached value is non-zero: this pins the
# parts the special cases above zero out -- the rotation of q, the stacking
# of the attention and feed-forward blocks over several layers, and the
# cache written by one step and read by the next.
SPEC_TYPES = dict(tok=O.Q8_0, wq=O.Q8_0, wk=O.Q4_0, wv=O.Q6_K, wo=O.Q4_0, gate=O.Q8_0, up=O.Q6_K,
                  down=O.Q4_0, out=O.Q6_K)


def _spec_model(cfg, w, kk, vv):
    from . import spec_np
    qt = lambda q: (q.type, q.data)
    weights = dict(tok_embd=qt(w.tok_embd), output=qt(w.output), output_norm=w.output_norm,
                   layers=[dict(attn_norm=L.attn_norm, ffn_norm=L.ffn_norm,
                                **{k: qt(getattr(L, k)) for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up",
                                                                   "w_down")}) for L in w.layers])
    c = dict(n_layers=cfg.n_layers, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
             head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, ctx_cap=cfg.ctx_cap, rms_eps=cfg.rms_eps,
             rope_theta=cfg.rope_theta)
    return spec_np.SpecModel(c, weights, kk.view(np.float16), vv.view(np.float16))


@pytest.mark.parametrize("n_q_heads,n_kv_heads", [(4, 2), (8, 2)])
def test_decode_step_matches_an_independent_numpy_reading(n_q_heads, n_kv_heads):
    cfg = tiny_config(n_layers=3, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, rope_theta=10000.0)
    w = build_oracle_model(cfg, seed=8, wtype=SPEC_TYPES)
    n_pos = 6
    kk = np.stack([synth.kv_prefix_bits(8, l, 0, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    vv = np.stack([synth.kv_prefix_bits(8, l, 1, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    spec = _spec_model(cfg, w, kk, vv)
    dec = O.Decoder(cfg, w, kk.copy(), vv.copy())
    # every weight matrix has non-zero entries, every gain differs from 1
    for L in w.layers:
        assert np.any(L.attn_norm != 1) and np.any(L.ffn_norm != 1)
        for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            assert np.count_nonzero(getattr(L, k).data) > 0
    tok_o = tok_s = 5
    for s in range(4):
        ref, nxt_s = spec.step(tok_s, n_pos + s)
        got, nxt_o = dec.step(tok_o, n_pos + s)
        scale = np.abs(ref).max()
        assert np.abs(got - ref).max() <= 1e-12 * scale, f"step {s}: {np.abs(got - ref).max() / scale:.2e}"
        assert nxt_o == nxt_s, f"step {s}"
        # the cache both wrote at slot pos holds the same fp16 values
        assert np.array_equal(dec.kv_k[:, :, n_pos + s, :], spec.k[:, :, n_pos + s, :].view(np.uint16))
        assert np.array_equal(dec.kv_v[:, :, n_pos + s, :], spec.v[:, :, n_pos + s, :].view(np.uint16))
        tok_o, tok_s = nxt_o, nxt_s


def test_spec_reading_sees_a_dropped_query_rotation():
    """The numpy reading is sharp enough to catch the mistake the special
    cases cannot: the same step without RoPE on q differs well beyond the
    tolerance above."""
    from . import spec_np
    cfg = tiny_config(n_layers=2, rope_theta=10000.0)
    w = build_oracle_model(cfg, seed=9, wtype=SPEC_TYPES)
    n_pos = 6
    kk = np.stack([synth.kv_prefix_bits(9, l, 0, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    vv = np.stack([synth.kv_prefix_bits(9, l, 1, cfg.n_kv_heads, cfg.ctx_cap, cfg.head_dim, n_pos)
                   for l in range(cfg.n_layers)])
    dec = O.Decoder(cfg, w, kk.copy(), vv.copy())
    got, _ = dec.step(5, n_pos)
    spec = _spec_model(cfg, w, kk, vv)
    rope = spec_np.rope
    assert cfg.n_q_heads != cfg.n_kv_heads

    def rope_k_only(v, n_heads, d, pos, theta):     # the q heads pass unrotated
        return v if n_heads == cfg.n_q_heads else rope(v, n_heads, d, pos, theta)

    spec_np.rope = rope_k_only
    try:
        bad, _ = spec.step(5, n_pos)
    finally:
        spec_np.rope = rope
    assert np.abs(got - bad).max() > 1e-6 * np.abs(got).max()
