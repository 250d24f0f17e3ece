"""Decode parity at the benchmark's own models, checked against the oracle.

The models are built on the device by devmodel.build exactly as bench.py
builds them (seeded N(0, 0.02) values from torch's generator encoded by
nt_quantize, gains 1, a prefilled N(0, 1) fp16 KV cache from torch's
generator).  The oracle's model takes none of the library's bytes: the same
seeded values are drawn again, copied to the host and encoded by the
oracle's own encoder; each matrix the device holds must equal the oracle's
encoding byte for byte, and the oracle decodes its own bytes over the same
fp16 cache prefix.

* Llama-3-8B shape, Q8_0 throughout (the write-up's "Roadmap", phase 1: Llama
  8B Q8_0): all 32 layers, the full 128256-row head, 16 greedy tokens from
  position 1024 in the captured-graph mode the benchmark times.
* Llama-70B shape, Q4_K with Q6_K for attn_v, ffn_down and the head (the
  write-up's "Performance" section runs 70B Q4_K_M): all 80 layers and the
  full 128256 x 8192 Q6_K head, 4 greedy tokens from position 4096.

Protocol: tests/parity_util.py.  The oracle runs on 16 host threads; the 70B
case needs about 45 GB of host memory for the oracle's copy of the weights.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_decode_dequant_amd import devmodel, nt, workloads

from .parity_util import greedy_parity_run

pytestmark = pytest.mark.gpu


THREADS = 16


def oracle_bytes(rows, cols, t, sid, dev):
    """The oracle's encoding of devmodel's seeded values for one matrix,
    chunks split over THREADS host threads at block boundaries."""
    rb = O.row_bytes(t, cols)
    out = np.empty(rows * rb, np.uint8)
    be, bb = O.block_elems(t), O.block_bytes(t)
    with ThreadPoolExecutor(THREADS) as pool:
        for r0, n, w in devmodel.value_chunks(rows, cols, 0, sid, dev):
            v = w.cpu().numpy()
            nb = v.size // be
            cuts = [nb * i // THREADS for i in range(THREADS + 1)]
            base = r0 * rb

            def enc(i):
                lo, hi = cuts[i], cuts[i + 1]
                if hi > lo:
                    out[base + lo * bb:base + hi * bb] = O.quantize(t, v[lo * be:hi * be])

            list(pool.map(enc, range(THREADS)))
    return out


def oracle_decoder(shape, extra, say=print):
    """An oracle.Decoder over the oracle's own encoding of the model's values;
    every matrix of the device model must equal it byte for byte."""
    w = extra["weights"]
    dev = extra["k_cache"].device
    host = {}
    for l, name, rows, cols, t, sid in devmodel.matrix_specs(shape):
        if l is not None and name == "wq" and l % 10 == 0:
            say(f"  oracle encoding: layer {l} of {shape.n_layers}")
        ob = oracle_bytes(rows, cols, t, sid, dev)
        d = (w[name] if l is None else w["layers"][l][name])[1]
        assert torch.equal(d, torch.from_numpy(ob).to(dev)), f"layer {l} {name}: device bytes differ from the oracle's"
        host[(l, name)] = O.QTensor(int(t), ob)
    qt = lambda l, name: host[(l, name)]
    f32 = lambda t: t.cpu().numpy().astype(np.float32)
    layers = [O.LayerWeights(attn_norm=f32(L["attn_norm"]), ffn_norm=f32(L["ffn_norm"]),
                             **{k: qt(l, k) for k in nt.Model.MATS}) for l, L in enumerate(w["layers"])]
    mw = O.ModelWeights(tok_embd=qt(None, "tok_embd"), output_norm=f32(w["output_norm"]),
                        output=qt(None, "output"), layers=layers)
    cfg = O.Config(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                   shape.vocab, shape.ctx_cap, shape.rms_eps, shape.rope_theta)
    kk = np.ascontiguousarray(extra["k_cache"].cpu().numpy().view(np.uint16))
    vv = np.ascontiguousarray(extra["v_cache"].cpu().numpy().view(np.uint16))
    return O.Decoder(cfg, mw, kk, vv)


def _bench_model_parity(shape, n_steps, what, capfd):
    """Runs for minutes (the oracle encodes and decodes the whole model on the
    host), so its progress goes straight to the terminal, past pytest's
    output capture."""
    def say(msg):
        with capfd.disabled():
            print(msg, flush=True)

    say(f"{what}: building {shape.name} on the device")
    model, extra = devmodel.build(shape)
    torch.cuda.synchronize()
    dec = oracle_decoder(shape, extra, say)
    say(f"{what}: oracle encoding done, equal to the device bytes; decoding")
    try:
        r = greedy_parity_run(model, dec, shape.vocab, shape.ctx, 1, n_steps, what=what, graph=True,
                              oracle_threads=16, say=say)
    finally:
        model.close()
        del model, extra, dec
        torch.cuda.empty_cache()
    return r


@pytest.mark.timeout(900)
def test_llama8b_q8_0_benchmark_model_full_depth(capfd):
    _bench_model_parity(workloads.LLAMA_8B_Q8_0, 16, "8B Q8_0 (32 layers)", capfd)


@pytest.mark.timeout(900)
def test_llama70b_mix_benchmark_model_full_depth(capfd):
    _bench_model_parity(workloads.LLAMA_70B_MIX, 4, "70B Q4_K/Q6_K (80 layers)", capfd)
