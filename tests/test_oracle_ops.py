"""Pins for the oracle's fp64 ops: closed forms, invariants, special cases and
library routines -- never the oracle against a retyped copy of itself.

The ops are the kernels the ntransformer write-up (GeekNews topic 26894)
names in "Architecture" (GEMV, RMSNorm, RoPE, SwiGLU, softmax) and the Llama
pieces of "Main features" (GQA attention over the F16 KV cache of
"Roadmap").
"""
import math

import numpy as np
import pytest

import oracle as O
from block_quantized_decode_dequant_amd import synth

TYPES = [O.Q8_0, O.Q4_0, O.Q4_K, O.Q6_K]
TID = ["q8_0", "q4_0", "q4_k", "q6_k"]


def _matrix(t, rows, cols, seed=0):
    w = synth.normal_f32(seed, 40 + t, rows * cols, std=0.02)
    return O.quantize(t, w)


# ---- GEMV ------------------------------------------------------------------
def test_gemv_one_hot_selects_exactly():
    """Q8_0 rows with d = 1 and a single code 1 pick one x value, exactly."""
    rows, cols = 48, 96
    cols_pick = synth.uniform_int(0, 50, rows, 0, cols - 1)
    qs = np.zeros((rows, cols), np.int8)
    qs[np.arange(rows), cols_pick] = 1
    d = np.full(rows * cols // 32, 0x3C00, np.uint16)
    W = O.pack_q8_0(d, qs)
    x = synth.normal_f32(0, 51, cols)
    y = O.gemv(O.Q8_0, W, rows, cols, x)
    assert np.array_equal(y, x[cols_pick].astype(np.float64))


@pytest.mark.parametrize("t", TYPES, ids=TID)
def test_gemv_matches_numpy_matmul(t):
    """A library fp64 product over the decoded weights (decoders pinned
    separately) agrees to fp64 rounding."""
    rows, cols = 37, 512
    W = _matrix(t, rows, cols)
    x = synth.normal_f32(0, 52, cols)
    y = O.gemv(t, W, rows, cols, x)
    w = O.dequant(t, W, rows * cols).astype(np.float64).reshape(rows, cols)
    ref = w @ x.astype(np.float64)
    scale = np.abs(w) @ np.abs(x.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 1e-13 * scale + 1e-300)


@pytest.mark.parametrize("t", TYPES, ids=TID)
def test_gemv_linear_in_x_and_thread_invariant(t):
    rows, cols = 64, 256
    W = _matrix(t, rows, cols, seed=1)
    x = synth.normal_f32(1, 53, cols).astype(np.float64)
    y1 = O.gemv(t, W, rows, cols, x, nthreads=1)
    y8 = O.gemv(t, W, rows, cols, x, nthreads=7)
    assert np.array_equal(y1, y8)
    assert np.array_equal(O.gemv(t, W, rows, cols, 4.0 * x), 4.0 * y1)      # power of 2: exact
    x2 = synth.normal_f32(1, 54, cols).astype(np.float64)
    y2 = O.gemv(t, W, rows, cols, x2)
    ys = O.gemv(t, W, rows, cols, x + x2)
    assert np.allclose(ys, y1 + y2, rtol=1e-12, atol=1e-12)
    ids = np.array([63, 0, 17, 17, 5])
    assert np.array_equal(O.gemv_rows(t, W, rows, cols, x, ids), y1[ids])


def test_gemv_rejects_ragged_columns():
    with pytest.raises(ValueError):
        O.gemv(O.Q4_K, np.zeros(1000, np.uint8), 2, 100, np.zeros(100))


# ---- RMSNorm -------------------------------------------------------------------
def test_rmsnorm_closed_forms():
    n, eps = 4096, 1e-5
    x = synth.normal_f32(0, 60, n).astype(np.float64)
    one = np.ones(n)
    y = O.rmsnorm(x, one, eps)
    m = np.mean(x * x)
    assert math.isclose(np.mean(y * y), m / (m + eps), rel_tol=1e-12)
    assert np.allclose(y / x, 1 / math.sqrt(m + eps), rtol=1e-14)
    c = np.full(64, 0.5)
    assert np.allclose(O.rmsnorm(c, one[:64], eps), 0.5 / math.sqrt(0.25 + eps), rtol=1e-15)
    g = synth.normal_f32(0, 61, n, mean=1.0, std=0.1).astype(np.float64)
    assert np.allclose(O.rmsnorm(x, g, eps), g * y, rtol=1e-15)          # linear in the gain
    y0 = O.rmsnorm(x, one, 0.0)
    assert np.allclose(O.rmsnorm(1000.0 * x, one, 0.0), y0, rtol=1e-13)  # scale invariant at eps=0


def test_rmsnorm_eps_inside_root():
    """For x = 0 except one entry, eps placement is visible: y = x/sqrt(x^2/n + eps)."""
    x = np.zeros(4)
    x[2] = 2.0
    y = O.rmsnorm(x, np.ones(4), 0.5)
    assert math.isclose(y[2], 2.0 / math.sqrt(4.0 / 4 + 0.5), rel_tol=1e-15)


# ---- RoPE ------------------------------------------------------------------------
def test_rope_position_zero_is_identity():
    v = synth.normal_f32(0, 62, 4 * 128).astype(np.float64)
    assert np.array_equal(O.rope(v, 4, 128, 0, 500000.0), v)


def test_rope_first_pair_turns_by_one_radian_at_pos_one():
    v = np.zeros(2 * 128)
    v[0] = 1.0          # head 0, pair 0
    v[128 + 2] = 1.0    # head 1, pair 1
    r = O.rope(v, 2, 128, 1, 500000.0)
    assert math.isclose(r[0], math.cos(1.0), rel_tol=1e-15)
    assert math.isclose(r[1], math.sin(1.0), rel_tol=1e-15)
    ang = 500000.0 ** (-1.0 / 64)    # pair i=1 turns by theta^(-2/128) at pos 1
    assert math.isclose(r[128 + 2], math.cos(ang), rel_tol=1e-14)
    assert math.isclose(r[128 + 3], math.sin(ang), rel_tol=1e-14)
    assert np.count_nonzero(r) == 4


def test_rope_norms_and_relative_positions():
    H, D, th = 3, 128, 500000.0
    q = synth.normal_f32(0, 63, H * D).astype(np.float64)
    k = synth.normal_f32(0, 64, H * D).astype(np.float64)
    rq = O.rope(q, H, D, 777, th)
    pair = lambda a: np.hypot(a[0::2], a[1::2])
    assert np.allclose(pair(rq), pair(q), rtol=1e-13)
    # <R_m q, R_n k> depends only on m - n
    a = np.dot(O.rope(q, H, D, 1000, th), O.rope(k, H, D, 990, th))
    b = np.dot(O.rope(q, H, D, 10, th), k)
    assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)
    # rotating by 3 then by 4 equals rotating by 7
    assert np.allclose(O.rope(O.rope(q, H, D, 3, th), H, D, 4, th), O.rope(q, H, D, 7, th),
                       rtol=1e-12, atol=1e-13)


# ---- softmax ---------------------------------------------------------------------
def test_softmax_invariants_and_closed_forms():
    s = synth.normal_f32(0, 65, 1000, std=3.0).astype(np.float64)
    p = O.softmax(s)
    assert math.isclose(p.sum(), 1.0, rel_tol=1e-14) and np.all(p > 0)
    assert np.allclose(O.softmax(s + 123.0), p, rtol=1e-12)
    assert np.allclose(O.softmax(np.full(7, 2.5)), 1 / 7, rtol=1e-15)
    a, b = 1.3, -0.4
    p2 = O.softmax(np.array([a, b]))
    assert math.isclose(p2[0], 1 / (1 + math.exp(b - a)), rel_tol=1e-15)
    big = O.softmax(np.array([1000.0, 999.0]))
    assert math.isclose(big[0], 1 / (1 + math.exp(-1.0)), rel_tol=1e-15)
    assert int(np.argmax(p)) == int(np.argmax(s))


# ---- SwiGLU / SiLU --------------------------------------------------------------
def test_silu_identities():
    for a in [-7.5, -1.0, -0.1, 0.3, 2.0, 11.0]:
        assert math.isclose(O.silu(a) - O.silu(-a), a, rel_tol=1e-14, abs_tol=1e-15)
    assert O.silu(0.0) == 0.0
    assert math.isclose(O.silu(math.log(3.0)), 0.75 * math.log(3.0), rel_tol=1e-15)
    assert abs(O.silu(-60.0)) < 1e-24
    g = synth.normal_f32(0, 66, 100, std=2.0).astype(np.float64)
    u = synth.normal_f32(0, 67, 100).astype(np.float64)
    out = O.swiglu(g, u)
    assert np.allclose(O.swiglu(g, np.ones(100)) * u, out, rtol=1e-15)
    assert np.all(np.sign(O.swiglu(g, np.ones(100))) == np.sign(g))


# ---- argmax -------------------------------------------------------------------------
def test_argmax_lowest_index_on_ties():
    assert O.argmax(np.array([1.0, 5.0, 5.0, -2.0])) == 1
    assert O.argmax(np.array([-3.0, -1.0, -1.0])) == 1
    assert O.argmax(np.array([4.0])) == 0
    v = synth.normal_f32(0, 68, 128256).astype(np.float64)
    assert O.argmax(v) == int(np.argmax(v))


# ---- attention -----------------------------------------------------------------------
def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def _cache(n_kv, ctx, D, n_pos, seed, which):
    return synth.kv_prefix_bits(seed, 0, which, n_kv, ctx, D, n_pos)


def test_attention_single_slot_returns_v():
    Hq, Hkv, D, ctx = 8, 2, 64, 4
    kc = np.zeros((Hkv, ctx, D), np.uint16)
    vc = np.zeros((Hkv, ctx, D), np.uint16)
    q = synth.normal_f32(0, 70, Hq * D)
    kn = synth.normal_f32(0, 71, Hkv * D)
    vn = synth.normal_f32(0, 72, Hkv * D)
    o = O.attention(q, kn, vn, kc, vc, Hq, Hkv, D, ctx, 0).reshape(Hq, D)
    vn16 = _f16(vn).reshape(Hkv, D)
    for h in range(Hq):
        assert np.allclose(o[h], vn16[h // 4], rtol=1e-15, atol=0)
    # the new k and v were stored at slot 0, rounded to fp16 (numpy's IEEE cast)
    assert np.array_equal(kc[:, 0, :].reshape(-1), kn.astype(np.float16).view(np.uint16))
    assert np.array_equal(vc[:, 0, :].reshape(-1), vn.astype(np.float16).view(np.uint16))


def test_attention_equal_keys_average_values_and_ignore_later_slots():
    Hq, Hkv, D, ctx, pos = 4, 2, 32, 16, 9
    key = synth.normal_f32(0, 73, D).astype(np.float16).view(np.uint16)
    kc = np.tile(key, (Hkv, ctx, 1)).astype(np.uint16)
    vc = _cache(Hkv, ctx, D, pos, 0, 1)
    vc[:, pos + 1:, :] = 0x7E00          # NaN beyond pos must never be read
    kc[:, pos + 1:, :] = 0x7E00
    kn = np.tile(key.view(np.float16).astype(np.float64), Hkv)
    vn = synth.normal_f32(0, 74, Hkv * D)
    q = synth.normal_f32(0, 75, Hq * D)
    o = O.attention(q, kn, vn, kc, vc, Hq, Hkv, D, ctx, pos).reshape(Hq, D)
    vals = vc.view(np.float16).astype(np.float64)
    for h in range(Hq):
        g = h // 2
        assert np.allclose(o[h], vals[g, : pos + 1].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_two_slots_closed_form_and_groups():
    Hq, Hkv, D, ctx = 4, 2, 16, 8
    kc = np.zeros((Hkv, ctx, D), np.uint16)
    vc = np.zeros((Hkv, ctx, D), np.uint16)
    k0 = np.zeros(D); k0[0] = 1.0
    v0 = np.arange(D, dtype=np.float64) / 8
    kc[:, 0] = k0.astype(np.float16).view(np.uint16)
    vc[:, 0] = v0.astype(np.float16).view(np.uint16)
    k1 = np.zeros(Hkv * D); k1[1] = 1.0; k1[D + 1] = 1.0
    v1 = -np.tile(np.ones(D), Hkv); v1[D:] = 3.0
    q = np.zeros(Hq * D)
    q[0], q[1] = 2.0, -1.0         # head 0: s0 = 2/4, s1 = -1/4  (scale 1/sqrt(16))
    q[D + 0], q[D + 1] = 2.0, -1.0  # head 1 equals head 0 (same group)
    q[2 * D + 1] = 4.0             # head 2 (group 1): s0 = 0, s1 = 1
    o = O.attention(q, np.zeros(Hkv * D) + k1, v1, kc, vc, Hq, Hkv, D, ctx, 1).reshape(Hq, D)
    p0 = 1 / (1 + math.exp(-0.25 - 0.5))
    assert np.allclose(o[0], p0 * v0 + (1 - p0) * (-1.0), rtol=1e-14)
    assert np.array_equal(o[0], o[1])
    p0b = 1 / (1 + math.exp(1.0))
    assert np.allclose(o[2], p0b * v0 + (1 - p0b) * 3.0, rtol=1e-14)
    assert np.allclose(o[3], 0.5 * v0 + 0.5 * 3.0, rtol=1e-14)   # q = 0: uniform weights


def test_attention_rejects_bad_shapes():
    kc = np.zeros((2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        O.attention(np.zeros(24), np.zeros(16), np.zeros(16), kc, kc.copy(), 3, 2, 8, 4, 0)
    with pytest.raises(ValueError):
        O.attention(np.zeros(32), np.zeros(16), np.zeros(16), kc, kc.copy(), 4, 2, 8, 4, 4)


@pytest.mark.parametrize("t", [O.Q8_0, O.Q4_K, O.Q6_K])
def test_gemm_batch_is_the_dequantized_matrix_product(t):
    # k vectors against one matrix: the decoded matrix times X (numpy, fp64),
    # and each row of the result is that vector's own product (no mixing)
    rows, cols, k = 9, 512, 3
    W = O.quantize(t, synth.normal_f32(21, t, rows * cols, std=0.05))
    X = np.stack([synth.normal_f32(22, 10 * t + n, cols) for n in range(k)])
    Y = O.gemm_batch(t, W, rows, cols, X)
    Wd = O.dequant(t, W, rows * cols).astype(np.float64).reshape(rows, cols)
    assert Y.shape == (k, rows)
    np.testing.assert_allclose(Y, X.astype(np.float64) @ Wd.T, rtol=1e-12, atol=1e-12)
    X2 = X.copy()
    X2[1] = 0.0
    Y2 = O.gemm_batch(t, W, rows, cols, X2)
    assert np.all(Y2[1] == 0.0) and np.array_equal(Y2[[0, 2]], Y[[0, 2]])
