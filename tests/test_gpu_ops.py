"""GPU parity for RMSNorm, RoPE, softmax, SwiGLU, argmax, embedding lookup and
decode attention against the fp64 oracle on the same seeded inputs.

Bars: the embedding row and the fp16 cache entries are bit-exact; argmax is
exact (lowest index on ties); float outputs within 1e-4 + 2e-3 |ref|.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_decode_dequant_amd import nt, synth

from .gpu_util import assert_close, device, host, to_dev

pytestmark = pytest.mark.gpu


def _i32(v):
    return torch.tensor([v], dtype=torch.int32, device=device())


@pytest.mark.parametrize("n", [1, 255, 4096, 5000, 8192])
def test_rmsnorm(n):
    x = synth.normal_f32(5, 500, n, std=3.0)
    g = synth.normal_f32(5, 501, n, mean=1.0, std=0.1)
    y = torch.empty(n, dtype=torch.float32, device=device())
    nt.nt_rmsnorm(to_dev(x), to_dev(g), y, n, 1e-5)
    assert_close(host(y), O.rmsnorm(x, g, 1e-5), what="rmsnorm")


def test_rmsnorm_in_place():
    n = 4096
    x = synth.normal_f32(5, 502, n)
    g = np.ones(n, np.float32)
    dx = to_dev(x)
    nt.nt_rmsnorm(dx, to_dev(g), dx, n, 1e-5)
    assert_close(host(dx), O.rmsnorm(x, g, 1e-5), what="rmsnorm in place")


@pytest.mark.parametrize("pos", [0, 1, 777, 1151, 4159])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (64, 8, 128), (4, 2, 64)])
def test_rope(pos, hq, hkv, d):
    q = synth.normal_f32(6, 510, hq * d)
    k = synth.normal_f32(6, 511, hkv * d)
    dq, dk = to_dev(q), to_dev(k)
    nt.nt_rope(dq, dk, hq, hkv, d, _i32(pos), 500000.0)
    assert_close(host(dq), O.rope(q, hq, d, pos, 500000.0), what="rope q")
    assert_close(host(dk), O.rope(k, hkv, d, pos, 500000.0), what="rope k")


@pytest.mark.parametrize("n", [1, 7, 1025, 128256])
def test_softmax(n):
    s = synth.normal_f32(7, 520, n, std=3.0)
    ds = to_dev(s)
    nt.nt_softmax(ds, n)
    assert_close(host(ds), O.softmax(s), what="softmax")


@pytest.mark.parametrize("n", [1, 14336, 28672, 1000])
def test_swiglu(n):
    g = synth.normal_f32(8, 530, n, std=2.0)
    u = synth.normal_f32(8, 531, n)
    out = torch.empty(n, dtype=torch.float32, device=device())
    nt.nt_swiglu(to_dev(g), to_dev(u), out, n)
    assert_close(host(out), O.swiglu(g, u), what="swiglu")


def test_argmax_ties_and_edges():
    v = synth.normal_f32(9, 540, 128256)
    out = _i32(-1)
    nt.nt_argmax(to_dev(v), v.size, out)
    assert int(host(out)[0]) == O.argmax(v)
    w = v.copy()
    top = np.float32(v.max() + 1)
    w[90000] = top
    w[70001] = top                      # two equal maxima: the lower index wins
    nt.nt_argmax(to_dev(w), w.size, out)
    assert int(host(out)[0]) == 70001 == O.argmax(w)
    z = np.full(1000, -np.inf, np.float32)
    nt.nt_argmax(to_dev(z), z.size, out)
    assert int(host(out)[0]) == 0
    one = np.array([3.5], np.float32)
    nt.nt_argmax(to_dev(one), 1, out)
    assert int(host(out)[0]) == 0


@pytest.mark.parametrize("t", [O.Q8_0, O.Q4_0, O.Q4_K, O.Q5_K, O.Q6_K], ids=["q8_0", "q4_0", "q4_k", "q5_k", "q6_k"])
def test_embed_row_bit_exact(t):
    vocab, hidden = 300, 1024
    table = O.quantize(t, synth.normal_f32(10, 550 + t, vocab * hidden, std=0.02))
    dt = to_dev(table)
    out = torch.empty(hidden, dtype=torch.float32, device=device())
    rb = O.row_bytes(t, hidden)
    for tok in (0, 137, vocab - 1):
        nt.nt_embed(t, dt, vocab, hidden, _i32(tok), out)
        ref = O.dequant(t, table[tok * rb:(tok + 1) * rb], hidden)
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))
    nt.nt_embed(t, dt, vocab, hidden, _i32(vocab), out)      # out of range: NaN, no read
    assert np.all(np.isnan(host(out)))


# ---- attention ------------------------------------------------------------------
ATTN_CASES = [
    # hq, hkv, d, ctx_cap, pos
    (32, 8, 128, 1152, 1024), (32, 8, 128, 1152, 0), (32, 8, 128, 1152, 1151), (32, 8, 128, 1152, 31),
    (32, 8, 128, 1152, 32), (64, 8, 128, 4160, 4096), (64, 8, 128, 4160, 4159), (4, 2, 64, 32, 17),
    (8, 8, 64, 64, 63), (16, 8, 128, 300, 150),
    # long context: the chunk reaches its 128-position cap, 128 chunks per kv head
    (32, 8, 128, 16384, 16000),
]


def _attn_inputs(hq, hkv, d, ctx, pos, seed):
    kc = synth.kv_prefix_bits(seed, 0, 0, hkv, ctx, d, pos)
    vc = synth.kv_prefix_bits(seed, 0, 1, hkv, ctx, d, pos)
    q = synth.normal_f32(seed, 560, hq * d)
    kn = synth.normal_f32(seed, 561, hkv * d)
    vn = synth.normal_f32(seed, 562, hkv * d)
    return q, kn, vn, kc, vc


@pytest.mark.parametrize("hq,hkv,d,ctx,pos", ATTN_CASES)
def test_attention_decode(hq, hkv, d, ctx, pos):
    q, kn, vn, kc, vc = _attn_inputs(hq, hkv, d, ctx, pos, seed=pos + ctx)
    desc = nt.attn_desc(hq, hkv, d, ctx)
    ws = torch.empty(nt.nt_attn_workspace_bytes(desc), dtype=torch.uint8, device=device())
    dk, dv = to_dev(kc), to_dev(vc)
    out = torch.empty(hq * d, dtype=torch.float32, device=device())
    nt.nt_attn_decode(desc, to_dev(q), to_dev(kn), to_dev(vn), dk, dv, _i32(pos), out, ws)
    ref = O.attention(q, kn, vn, kc, vc, hq, hkv, d, ctx, pos)    # updates kc, vc too
    assert_close(host(out), ref, what="attention")
    assert np.array_equal(host(dk), kc) and np.array_equal(host(dv), vc)


ROPE_CASES = [(32, 8, 128, 1152, 1024), (64, 8, 128, 4160, 4100), (4, 2, 64, 96, 70), (8, 8, 64, 64, 5),
              (16, 8, 128, 300, 299)]


@pytest.mark.parametrize("hq,hkv,d,ctx,pos", ROPE_CASES)
def test_attention_with_rope(hq, hkv, d, ctx, pos):
    """rope_theta > 0: q and the new k are rotated inside the kernel, exactly
    what nt_rope followed by nt_attn_decode computes; q is left untouched."""
    theta = 500000.0
    q, kn, vn, kc, vc = _attn_inputs(hq, hkv, d, ctx, pos, seed=pos + 2 * ctx)
    desc = nt.attn_desc(hq, hkv, d, ctx, rope_theta=theta)
    ws = torch.empty(nt.nt_attn_workspace_bytes(desc), dtype=torch.uint8, device=device())
    dq, dk, dv = to_dev(q), to_dev(kc), to_dev(vc)
    out = torch.empty(hq * d, dtype=torch.float32, device=device())
    nt.nt_attn_decode(desc, dq, to_dev(kn), to_dev(vn), dk, dv, _i32(pos), out, ws)
    qr = O.rope(q, hq, d, pos, theta)
    knr = O.rope(kn, hkv, d, pos, theta)
    ref = O.attention(qr, knr, vn, kc, vc, hq, hkv, d, ctx, pos)    # updates kc, vc too
    assert_close(host(out), ref, what="attention with rope")
    assert np.array_equal(host(dq), q), "q was modified"
    # the stored k may differ from the oracle's by one fp16 step where the
    # fp32 rotation lands next to a rounding boundary
    got_k = host(dk).view(np.float16).astype(np.float64)
    ref_k = kc.view(np.float16).astype(np.float64)
    assert np.all(np.abs(got_k - ref_k) <= np.abs(ref_k) * 2.0 ** -10 + 2.0 ** -24)
    assert np.array_equal(host(dv), vc)


def test_attention_with_entry_already_cached_and_bad_pos():
    hq, hkv, d, ctx, pos = 32, 8, 128, 1152, 700
    q, kn, vn, kc, vc = _attn_inputs(hq, hkv, d, ctx, pos, seed=3)
    ref = O.attention(q, kn, vn, kc, vc, hq, hkv, d, ctx, pos)    # kc, vc now hold the entry
    desc = nt.attn_desc(hq, hkv, d, ctx)
    ws = torch.empty(nt.nt_attn_workspace_bytes(desc), dtype=torch.uint8, device=device())
    dk, dv = to_dev(kc), to_dev(vc)
    out = torch.empty(hq * d, dtype=torch.float32, device=device())
    nt.nt_attn_decode(desc, to_dev(q), None, None, dk, dv, _i32(pos), out, ws)
    assert_close(host(out), ref, what="attention (cached entry)")
    nt.nt_attn_decode(desc, to_dev(q), to_dev(kn), to_dev(vn), dk, dv, _i32(ctx), out, ws)
    assert np.all(np.isnan(host(out)))
    assert np.array_equal(host(dk), kc) and np.array_equal(host(dv), vc)


def test_attention_deterministic():
    hq, hkv, d, ctx, pos = 64, 8, 128, 4160, 3000
    q, kn, vn, kc, vc = _attn_inputs(hq, hkv, d, ctx, pos, seed=4)
    desc = nt.attn_desc(hq, hkv, d, ctx)
    ws = torch.empty(nt.nt_attn_workspace_bytes(desc), dtype=torch.uint8, device=device())
    outs = []
    for _ in range(2):
        out = torch.empty(hq * d, dtype=torch.float32, device=device())
        nt.nt_attn_decode(desc, to_dev(q), to_dev(kn), to_dev(vn), to_dev(kc), to_dev(vc), _i32(pos), out, ws)
        outs.append(host(out))
    assert np.array_equal(outs[0], outs[1])
