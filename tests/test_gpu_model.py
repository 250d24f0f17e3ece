"""GPU parity for the whole decode step against the oracle's decode step on
the same seeded model, KV prefix and tokens.

Protocol: tests/parity_util.py (logits normwise within 5e-3 of the oracle's
every step, identical greedy tokens but for counted near-ties, at most one
per 16 steps).  The captured HIP graph must reproduce eager execution bit for
bit, replay after replay; the host-streamed mode must reproduce resident
execution bit for bit and match the oracle; a model read from a GGUF file
must match the oracle too.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_decode_dequant_amd import nt, synth

from .gpu_util import device, host
from .model_util import build_oracle_model, kv_prefix, tiny_config
from .parity_util import greedy_parity_run

pytestmark = pytest.mark.gpu


def _dev_qt(q: O.QTensor):
    return (q.type, torch.from_numpy(np.ascontiguousarray(q.data)).to(device()))


def upload(cfg: O.Config, w: O.ModelWeights, kk: np.ndarray, vv: np.ndarray):
    dev = device()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    weights = {
        "tok_embd": _dev_qt(w.tok_embd), "output": _dev_qt(w.output), "output_norm": f32(w.output_norm),
        "layers": [{"attn_norm": f32(L.attn_norm), "ffn_norm": f32(L.ffn_norm),
                    **{k: _dev_qt(getattr(L, k)) for k in nt.Model.MATS}} for L in w.layers],
    }
    ncfg = nt.model_config(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                           cfg.vocab, cfg.ctx_cap, cfg.rms_eps, cfg.rope_theta)
    ws = torch.empty(nt.nt_model_workspace_bytes(ncfg), dtype=torch.uint8, device=dev)
    kc = torch.from_numpy(kk.copy()).to(dev)
    vc = torch.from_numpy(vv.copy()).to(dev)
    return nt.Model(ncfg, weights, kc, vc, ws), kc, vc


def greedy_parity(cfg, w, n_pos, first_token, n_steps, graph=True, what=""):
    kk, vv = kv_prefix(cfg, 7, n_pos)
    dec = O.Decoder(cfg, w, kk.copy(), vv.copy())
    model, kc, vc = upload(cfg, w, kk, vv)
    r = greedy_parity_run(model, dec, cfg.vocab, n_pos, first_token, n_steps, what=what, graph=graph)
    model.close()
    return r["near_ties"]


@pytest.mark.parametrize("wtype", [O.Q8_0, O.Q4_0, O.Q4_K, O.Q5_K, O.Q6_K, "mix"],
                         ids=["q8_0", "q4_0", "q4_k", "q5_k", "q6_k", "mix"])
def test_tiny_model_greedy_parity(wtype):
    cfg = tiny_config()
    w = build_oracle_model(cfg, seed=11, wtype=wtype)
    greedy_parity(cfg, w, n_pos=8, first_token=5, n_steps=6)


@pytest.mark.parametrize("graph", [True, False], ids=["graph", "eager"])
def test_wide_mix_model_uses_fused_paths_throughout(graph):
    """hidden 2048: q and k (Q4_K) and v (Q6_K) share one paired two-format
    launch; every other matrix takes a fused path too (Q6_K down with 4-byte
    copies)."""
    cfg = tiny_config(n_layers=2, hidden=2048, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=512)
    w = build_oracle_model(cfg, seed=15, wtype="mix")
    greedy_parity(cfg, w, n_pos=5, first_token=3, n_steps=4, graph=graph)


def test_tiny_model_eager_path():
    cfg = tiny_config(n_layers=3, n_q_heads=8, n_kv_heads=2)
    w = build_oracle_model(cfg, seed=12, wtype="mix")
    greedy_parity(cfg, w, n_pos=0, first_token=9, n_steps=4, graph=False)


def _run_steps(model, cfg, n_pos, token, n, between=None):
    dev = device()
    d_tok = torch.tensor([token], dtype=torch.int32, device=dev)
    d_pos = torch.tensor([n_pos], dtype=torch.int32, device=dev)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    out = []
    for s in range(n):
        with torch.cuda.stream(side):
            model.step(d_tok, d_pos, logits, d_tok)
        out.append(host(logits).copy())
        if between:
            between()
    return out, int(host(d_tok)[0])


def test_graph_replays_match_eager_bitwise():
    cfg = tiny_config(n_layers=2)
    w = build_oracle_model(cfg, seed=13, wtype=O.Q4_K)
    kk, vv = kv_prefix(cfg, 3, 4)
    m1, _, _ = upload(cfg, w, kk, vv)
    m1.set_graph(False)
    eager, t1 = _run_steps(m1, cfg, 4, 17, 6)
    m2, _, _ = upload(cfg, w, kk, vv)
    m2.set_graph(True)

    def noise():  # the program's own eager work between replays
        a = torch.randn(4096, device=device())
        torch.cuda.synchronize()
        return float((a * a).sum())

    graph, t2 = _run_steps(m2, cfg, 4, 17, 6, between=noise)
    for s, (a, b) in enumerate(zip(eager, graph)):
        assert np.array_equal(a, b), f"replay {s} differs from eager"
    assert t1 == t2
    m1.close()
    m2.close()


def _blob_bytes(cfg_nt, types):
    offs, nbytes = nt.nt_layer_blob_layout(cfg_nt, types)
    return offs, nbytes


def test_streamed_layers_match_resident_bitwise():
    cfg = tiny_config(n_layers=5)
    w = build_oracle_model(cfg, seed=14, wtype="mix")
    kk, vv = kv_prefix(cfg, 5, 6)
    res, _, _ = upload(cfg, w, kk, vv)
    res.set_graph(False)
    ref, _ = _run_steps(res, cfg, 6, 3, 5)
    res.close()

    first = 2
    st_model, _, _ = upload(cfg, w, kk, vv)
    dec = O.Decoder(cfg, w, kk.copy(), vv.copy())
    types = [getattr(w.layers[first], k).type for k in nt.Model.MATS]
    offs, nbytes = nt.nt_layer_blob_layout(st_model.cfg, types)
    blobs = []
    for L in w.layers[first:]:
        b = torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)
        for off, k in zip(offs, nt.Model.MATS):
            data = getattr(L, k).data
            b[off:off + data.size] = torch.from_numpy(data)
        blobs.append(b)
    dbuf = [torch.empty(nbytes, dtype=torch.uint8, device=device()) for _ in range(2)]
    copy_stream = torch.cuda.Stream()
    st_model.stream_layers(first, blobs, dbuf[0], dbuf[1], copy_stream)
    got = []
    # the streamed steps against the oracle (greedy, same protocol as the
    # resident parity tests), and bit for bit against the resident run
    greedy_parity_run(st_model, dec, cfg.vocab, 6, 3, 5, what="streamed", graph=False,
                      each_step=lambda s_, lg: got.append(lg.copy()))
    for s, (a, b) in enumerate(zip(ref, got)):
        assert np.array_equal(a, b), f"streamed step {s} differs from resident"
    stats = st_model.stream_stats()
    ns = cfg.n_layers - first
    assert stats["steps"] == 5 and stats["layers_streamed"] == 5 * ns
    assert stats["h2d_bytes"] == 5 * ns * nbytes
    assert stats["copy_ms"] > 0 and stats["compute_ms"] > 0 and stats["wall_ms"] > 0
    st_model.stream_layers(None, None, None, None, None)
    st_model.close()


def test_llama8b_shaped_two_layers_full_vocab():
    """Llama-3-8B shapes (hidden 4096, 32/8 heads, FFN 14336, vocab 128256,
    RoPE theta 5e5, KV prefix of 1024 positions) with two of its 32 layers."""
    cfg = O.Config(2, 4096, 32, 8, 128, 14336, 128256, 1152, 1e-5, 500000.0)
    w = build_oracle_model(cfg, seed=21, wtype=O.Q8_0, gains="one")
    greedy_parity(cfg, w, n_pos=1024, first_token=1, n_steps=3)


def test_llama70b_layer_shape_mixed_kquants():
    """One layer at the Llama-70B shape (hidden 8192, 64/8 heads of 128, FFN
    28672, RoPE theta 5e5) in the mixed recipe (Q4_K; Q6_K for attn_v,
    ffn_down and the head), KV prefix of 4096 positions in a 4160-slot cache:
    the paired Q4_K/Q6_K q/k/v launch at 8192 columns, the 28672-row SwiGLU
    launch, the 28672-column down projection and attention over 4097-4099
    positions, each in the launch configuration of the 70B benchmark model.
    (Vocabulary 2048 keeps the oracle's build within seconds.)"""
    cfg = O.Config(1, 8192, 64, 8, 128, 28672, 2048, 4160, 1e-5, 500000.0)
    w = build_oracle_model(cfg, seed=31, wtype="mix", gains="one")
    greedy_parity(cfg, w, n_pos=4096, first_token=1, n_steps=3)


def test_step_past_the_cache_and_with_a_bad_token():
    """Out-of-range device values: a step at pos == ctx_cap gives NaN logits
    and token 0, advances the position and leaves both caches (and a guard
    region after them) untouched; a token outside [0, vocab) gives NaN logits
    and token 0 and writes nothing past the caches."""
    cfg = tiny_config(n_layers=2, ctx_cap=16)
    w = build_oracle_model(cfg, seed=41, wtype=O.Q4_K)
    kk, vv = kv_prefix(cfg, 7, cfg.ctx_cap)
    dev = device()
    n, guard = kk.size, 4096
    # the caches, each followed by a guard region that must keep its pattern
    kcg = torch.full((n + guard,), 0x1234, dtype=torch.int16, device=dev)
    vcg = torch.full((n + guard,), 0x4321, dtype=torch.int16, device=dev)
    kcg[:n] = torch.from_numpy(kk.reshape(-1).view(np.int16).copy()).to(dev)
    vcg[:n] = torch.from_numpy(vv.reshape(-1).view(np.int16).copy()).to(dev)
    ncfg = nt.model_config(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                           cfg.vocab, cfg.ctx_cap, cfg.rms_eps, cfg.rope_theta)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    weights = {
        "tok_embd": _dev_qt(w.tok_embd), "output": _dev_qt(w.output), "output_norm": f32(w.output_norm),
        "layers": [{"attn_norm": f32(L.attn_norm), "ffn_norm": f32(L.ffn_norm),
                    **{k: _dev_qt(getattr(L, k)) for k in nt.Model.MATS}} for L in w.layers],
    }
    ws = torch.empty(nt.nt_model_workspace_bytes(ncfg), dtype=torch.uint8, device=dev)
    model = nt.Model(ncfg, weights, kcg[:n], vcg[:n], ws)
    before_k, before_v = kcg.clone(), vcg.clone()
    logits = torch.zeros(cfg.vocab, dtype=torch.float32, device=dev)
    d_tok = torch.tensor([3], dtype=torch.int32, device=dev)
    d_pos = torch.tensor([cfg.ctx_cap], dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        model.step(d_tok, d_pos, logits, d_tok)
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(logits)))
    assert int(host(d_tok)[0]) == 0 and int(host(d_pos)[0]) == cfg.ctx_cap + 1
    assert torch.equal(kcg, before_k) and torch.equal(vcg, before_v)
    # a token outside [0, vocab) at a valid position
    d_tok.fill_(cfg.vocab)
    d_pos.fill_(5)
    with torch.cuda.stream(side):
        model.step(d_tok, d_pos, logits, d_tok)
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(logits)))
    assert int(host(d_tok)[0]) == 0 and int(host(d_pos)[0]) == 6
    assert torch.equal(kcg[n:], before_k[n:]) and torch.equal(vcg[n:], before_v[n:])
    model.close()


def test_decode_from_a_gguf_file(tmp_path):
    """A model read from a GGUF file (written by the tests' writer from the
    oracle's blocks, loaded by libnt's reader and gguf_model.load_llama)
    matches the oracle's decode of the same weights, and decodes bit for bit
    like the same weights uploaded directly."""
    from block_quantized_decode_dequant_amd import gguf_model

    from .gguf_writer import llama_gguf

    cfg = tiny_config(n_layers=2, n_q_heads=8, n_kv_heads=2)
    w = build_oracle_model(cfg, seed=53, wtype="mix")
    path = tmp_path / "tiny.gguf"
    path.write_bytes(llama_gguf(cfg, w))
    gcfg, gweights = gguf_model.load_llama(str(path), ctx_cap=cfg.ctx_cap)
    assert (gcfg.n_layers, gcfg.hidden, gcfg.vocab, gcfg.ctx_cap) == (cfg.n_layers, cfg.hidden, cfg.vocab, cfg.ctx_cap)
    kk, vv = kv_prefix(cfg, 7, 8)
    direct, _, _ = upload(cfg, w, kk, vv)
    dev = device()
    ws = torch.empty(nt.nt_model_workspace_bytes(gcfg), dtype=torch.uint8, device=dev)
    kc = torch.from_numpy(kk.copy()).to(dev)
    vc = torch.from_numpy(vv.copy()).to(dev)
    from_file = nt.Model(gcfg, gweights, kc, vc, ws)
    a, ta = _run_steps(direct, cfg, 8, 5, 4)
    dec = O.Decoder(cfg, w, kk.copy(), vv.copy())
    b = []
    greedy_parity_run(from_file, dec, cfg.vocab, 8, 5, 4, what="gguf", graph=False,
                      each_step=lambda s_, lg: b.append(lg.copy()))
    for s, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"step {s}"
    direct.close()
    from_file.close()


def _host_blob(L, offs, nbytes):
    b = np.zeros(nbytes, np.uint8)
    for off, k in zip(offs, nt.Model.MATS):
        data = getattr(L, k).data
        b[off:off + data.size] = data
    return b


def _pinned_staging(nbytes):
    """Two pinned host buffers, 4096-byte aligned, of at least nbytes each."""
    s = (nbytes + 4095) // 4096 * 4096
    raw = torch.empty(2 * s + 4096, dtype=torch.uint8, pin_memory=True)
    lead = (-raw.data_ptr()) % 4096
    return raw, raw[lead:lead + s], raw[lead + s:lead + 2 * s]


def _three_tier(cfg, w, kk, vv, path, first_streamed, first_file, direct=True):
    """A model with layers [0, first_streamed) resident, [first_streamed,
    first_file) pinned, [first_file, n_layers) read from `path`."""
    from block_quantized_decode_dequant_amd import devmodel

    model, _, _ = upload(cfg, w, kk, vv)
    types = [getattr(w.layers[first_streamed], k).type for k in nt.Model.MATS]
    offs, nbytes = nt.nt_layer_blob_layout(model.cfg, types)
    blobs = []
    for L in w.layers[first_streamed:first_file]:
        b = torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)
        b.copy_(torch.from_numpy(_host_blob(L, offs, nbytes)))
        blobs.append(b)
    stride = devmodel.write_layer_file(path, (_host_blob(L, offs, nbytes) for L in w.layers[first_file:]), nbytes)
    dbuf = [torch.empty(nbytes, dtype=torch.uint8, device=device()) for _ in range(2)]
    keep, s0, s1 = _pinned_staging(nbytes)
    copy_stream = torch.cuda.Stream()
    model.stream_layers_tiered(first_streamed, blobs, dbuf[0], dbuf[1], copy_stream, str(path), first_file, 0,
                               stride, s0, s1, direct=direct)
    model._test_keep = [keep, blobs, dbuf]
    return model, nbytes, stride


@pytest.mark.parametrize("direct", [True, False], ids=["o_direct", "page_cache"])
def test_three_tiers_match_resident_and_the_oracle(tmp_path, direct):
    """Layers 0-1 resident, 2-3 from pinned host blobs, 4-6 read from a file
    each step (host-ordered: read, then copy, then compute): bit for bit the
    resident run, and the oracle's greedy decode."""
    cfg = tiny_config(n_layers=7)
    w = build_oracle_model(cfg, seed=16, wtype="mix")
    kk, vv = kv_prefix(cfg, 5, 6)
    res, _, _ = upload(cfg, w, kk, vv)
    res.set_graph(False)
    ref, _ = _run_steps(res, cfg, 6, 3, 5)
    res.close()
    model, nbytes, stride = _three_tier(cfg, w, kk, vv, tmp_path / "layers.bin", 2, 4, direct=direct)
    dec = O.Decoder(cfg, w, kk.copy(), vv.copy())
    got = []
    greedy_parity_run(model, dec, cfg.vocab, 6, 3, 5, what="three tiers", graph=False,
                      each_step=lambda s_, lg: got.append(lg.copy()))
    for s, (a, b) in enumerate(zip(ref, got)):
        assert np.array_equal(a, b), f"three-tier step {s} differs from resident"
    fs = model.file_stats()
    print(f"file tier: direct={fs['direct']} reads={fs['reads']} read_ms={fs['read_ms']:.3f}", flush=True)
    assert fs["file_layers"] == 3 and fs["reads"] == 5 * 3 and fs["read_bytes"] == 5 * 3 * nbytes
    st = model.stream_stats()
    assert st["layers_streamed"] == 5 * 5 and st["h2d_bytes"] == 5 * 5 * nbytes
    model.stream_layers(None, None, None, None, None)
    model.close()


def test_file_tier_read_failure_returns_eio_and_recovers(tmp_path):
    """A layer file cut short after the tier was enabled: the step's read of
    the missing blob fails, nt_decode_step returns NT_EIO having enqueued
    nothing that waits on it (the device still drains), the position does
    not advance; with the file restored the next step matches the oracle."""
    cfg = tiny_config(n_layers=4)
    w = build_oracle_model(cfg, seed=17, wtype=O.Q4_K)
    kk, vv = kv_prefix(cfg, 5, 6)
    path = tmp_path / "layers.bin"
    model, nbytes, stride = _three_tier(cfg, w, kk, vv, path, 1, 2, direct=False)
    full = path.read_bytes()
    with open(path, "r+b") as fh:
        fh.truncate(stride + nbytes // 2)       # the second file blob is cut in half
    dev = device()
    d_tok = torch.tensor([3], dtype=torch.int32, device=dev)
    d_pos = torch.tensor([6], dtype=torch.int32, device=dev)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    with pytest.raises(nt.NTError) as ei:
        with torch.cuda.stream(side):
            model.step(d_tok, d_pos, logits, d_tok)
    assert ei.value.status == nt.NT_EIO and "ends inside blob 1" in str(ei.value)
    torch.cuda.synchronize()                    # nothing queued waits on the failed read
    assert int(host(d_pos)[0]) == 6
    path.write_bytes(full)
    dec = O.Decoder(cfg, w, kk.copy(), vv.copy())
    greedy_parity_run(model, dec, cfg.vocab, 6, 3, 3, what="after recovery", graph=False)
    model.stream_layers(None, None, None, None, None)
    model.close()
