"""libnt's GGUF reader, on the CPU: files written by the tests' own writer
from the oracle's packed blocks are read back byte for byte with the Llama
configuration; malformed files are refused with an error and never read past
the end.  (No GGUF file made by another tool is available here: compatibility
with such files is checked against the published format only.)"""
import os
import struct

import numpy as np
import pytest

import oracle as O
from block_quantized_decode_dequant_amd import nt

from .gguf_writer import STR, U32, gguf_bytes, llama_gguf
from .model_util import build_oracle_model, tiny_config


def _write(tmp_path, data: bytes, name="m.gguf"):
    p = os.path.join(tmp_path, name)
    with open(p, "wb") as f:
        f.write(data)
    return p


@pytest.mark.parametrize("alignment", [32, 64])
def test_llama_file_round_trip(tmp_path, alignment):
    cfg = tiny_config(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512)
    w = build_oracle_model(cfg, seed=51, wtype="mix")
    path = _write(tmp_path, llama_gguf(cfg, w, ctx_len=777, alignment=alignment))
    with nt.GGUF(path) as g:
        c = g.llama_config()
        assert (c.n_layers, c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ffn, c.vocab, c.ctx_cap) == \
               (2, 256, 4, 2, 64, 512, cfg.vocab, 777)
        assert c.rms_eps == pytest.approx(cfg.rms_eps) and c.rope_theta == cfg.rope_theta
        assert g.llama_config(ctx_cap=40).ctx_cap == 40
        assert len(g) == 3 + 9 * cfg.n_layers
        t, r, cc, view = g.tensor("blk.1.ffn_down.weight")
        assert (t, r, cc) == (O.Q6_K, cfg.hidden, cfg.ffn)
        assert np.array_equal(view, w.layers[1].w_down.data)
        t, r, cc, view = g.tensor("blk.0.attn_q.weight")
        assert (t, r, cc) == (O.Q4_K, 4 * 64, 256) and np.array_equal(view, w.layers[0].wq.data)
        t, r, cc, view = g.tensor("output_norm.weight")
        assert (t, r, cc) == (0, 1, cfg.hidden)
        assert np.array_equal(view.view(np.float32), w.output_norm.astype(np.float32))
        with pytest.raises(KeyError):
            g.tensor("blk.9.attn_q.weight")


def test_tied_output_and_defaults(tmp_path):
    cfg = tiny_config(n_layers=1)
    w = build_oracle_model(cfg, seed=52, wtype=O.Q8_0)
    data = llama_gguf(cfg, w, tied_output=True)
    path = _write(tmp_path, data)
    with nt.GGUF(path) as g:
        assert "output.weight" not in g.names()
        assert g.llama_config().vocab == cfg.vocab


def test_head_size_keys(tmp_path):
    # without key_length the head size is hidden / heads; a value head size
    # other than the key head size is refused (one KV cache head size)
    cfg = tiny_config(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512)
    w = build_oracle_model(cfg, seed=53, wtype=O.Q8_0)
    with nt.GGUF(_write(tmp_path, llama_gguf(cfg, w, head_keys=False), name="nokeys.gguf")) as g:
        assert g.llama_config().head_dim == 64
    odd = llama_gguf(cfg, w, head_keys=False, extra_kv=[("llama.attention.key_length", U32, 64),
                                                        ("llama.attention.value_length", U32, 128)])
    with nt.GGUF(_write(tmp_path, odd, name="odd.gguf")) as g:
        with pytest.raises(nt.NTError) as e:
            g.llama_config()
        assert e.value.status == nt.NT_ESHAPE


def _minimal(kv=None, tensors=None, **kw):
    kv = kv if kv is not None else [("general.architecture", STR, "llama")]
    tensors = tensors if tensors is not None else [("x.weight", [32, 2], O.Q8_0, bytes(range(68)))]
    return gguf_bytes(kv, tensors, **kw)


def test_every_truncation_is_refused(tmp_path):
    data = _minimal()
    with nt.GGUF(_write(tmp_path, data)) as g:
        assert g.tensor("x.weight")[1:3] == (2, 32)
    for n in range(0, len(data) - 1):
        with pytest.raises(nt.NTError):
            nt.GGUF(_write(tmp_path, data[:n], name=f"t{n}.gguf"))


def test_malformed_headers_are_refused(tmp_path):
    good = _minimal()
    bad_magic = b"GGUG" + good[4:]
    bad_version = good[:4] + struct.pack("<I", 7) + good[8:]
    huge_count = good[:8] + struct.pack("<Q", 1 << 40) + good[16:]
    for i, data in enumerate([bad_magic, bad_version, huge_count]):
        with pytest.raises(nt.NTError):
            nt.GGUF(_write(tmp_path, data, name=f"b{i}.gguf"))
    # a tensor whose data runs past the end, and a misaligned tensor offset
    past = _minimal(tensors=[("x.weight", [32, 4], O.Q8_0, bytes(68))])   # 136 bytes declared, 68 given
    with pytest.raises(nt.NTError):
        nt.GGUF(_write(tmp_path, past, name="past.gguf"))
    # a tensor offset that breaks the alignment (the second tensor's 96 -> 100)
    two = _minimal(tensors=[("x.weight", [32, 2], O.Q8_0, bytes(68)), ("y.weight", [32, 1], O.Q8_0, bytes(34))])
    at = two.index(b"y.weight") + len(b"y.weight") + 4 + 2 * 8 + 4
    assert struct.unpack_from("<Q", two, at)[0] == 96
    misaligned = two[:at] + struct.pack("<Q", 100) + two[at + 8:]
    with pytest.raises(nt.NTError):
        nt.GGUF(_write(tmp_path, misaligned, name="mis.gguf"))
    # alignment that is not a power of two
    with pytest.raises(nt.NTError):
        nt.GGUF(_write(tmp_path, _minimal(kv=[("general.alignment", U32, 48)]), name="al.gguf"))


def test_unknown_tensor_type_is_reported_not_read(tmp_path):
    data = _minimal(tensors=[("q2.weight", [256, 1], 10, bytes(84)), ("x.weight", [32, 2], O.Q8_0, bytes(68))])
    with nt.GGUF(_write(tmp_path, data)) as g:
        assert g.tensor("x.weight")[0] == O.Q8_0
        with pytest.raises(nt.NTError) as e:
            g.tensor("q2.weight")
        assert e.value.status == nt.NT_ESHAPE


def test_llama_config_needs_the_llama_keys(tmp_path):
    with nt.GGUF(_write(tmp_path, _minimal(kv=[("general.architecture", STR, "gpt2")]))) as g:
        with pytest.raises(nt.NTError):
            g.llama_config(32)
    with nt.GGUF(_write(tmp_path, _minimal(), name="nokeys.gguf")) as g:
        with pytest.raises(nt.NTError):
            g.llama_config(32)
