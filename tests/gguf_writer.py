"""A plain GGUF v3 writer for the tests (test infrastructure): builds model
files from the oracle's packed blocks so the library's GGUF reader can be
checked.  Written from the published container definition:

    u32 magic "GGUF" | u32 version | u64 n_tensors | u64 n_kv
    n_kv x { string key | u32 type | value }
    n_tensors x { string name | u32 n_dims | u64 ne[n_dims] | u32 type | u64 offset }
    zero padding to the alignment | tensor data, each at an aligned offset

(string = u64 length + bytes; value types u8 0, i8 1, u16 2, i16 3, u32 4,
i32 5, f32 6, bool 7, string 8, array 9 (u32 element type, u64 count,
elements), u64 10, i64 11, f64 12; ne[0] is the fastest dimension.)
"""
from __future__ import annotations

import struct

import numpy as np

U8, I8, U16, I16, U32, I32, F32, BOOL, STR, ARR, U64, I64, F64 = range(13)
_FMT = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f", BOOL: "<?",
        U64: "<Q", I64: "<q", F64: "<d"}


def _str(s: str) -> bytes:
    b = s.encode()
    return struct.pack("<Q", len(b)) + b


def _value(t: int, v) -> bytes:
    if t == STR:
        return _str(v)
    if t == ARR:
        et, items = v
        out = struct.pack("<IQ", et, len(items))
        return out + b"".join(_value(et, x) for x in items)
    return struct.pack(_FMT[t], v)


def gguf_bytes(kv, tensors, alignment: int = 32, version: int = 3) -> bytes:
    """kv: list of (key, type, value); tensors: list of (name, ne, type, data
    bytes) with ne fastest-first.  Returns the file's bytes."""
    head = struct.pack("<IIQQ", 0x46554747, version, len(tensors), len(kv))
    head += b"".join(_str(k) + struct.pack("<I", t) + _value(t, v) for k, t, v in kv)
    infos, off, blobs = b"", 0, []
    for name, ne, t, data in tensors:
        infos += _str(name) + struct.pack("<I", len(ne)) + b"".join(struct.pack("<Q", n) for n in ne)
        infos += struct.pack("<IQ", t, off)
        blobs.append((off, bytes(data)))
        off = (off + len(data) + alignment - 1) // alignment * alignment
    meta = head + infos
    data_start = (len(meta) + alignment - 1) // alignment * alignment
    out = bytearray(meta + b"\0" * (data_start - len(meta)))
    for o, b in blobs:
        out += b"\0" * (data_start + o - len(out))
        out += b
    return bytes(out)


def llama_gguf(cfg, w, ctx_len: int = 4096, alignment: int = 32, tied_output: bool = False,
               extra_kv=(), head_keys: bool = True) -> bytes:
    """A Llama model file from an oracle model (cfg: oracle Config, w: its
    ModelWeights): llama.* keys, a small string-array vocabulary key, and the
    tensors under their GGUF names.  F32 norm gains.  head_keys=False leaves
    out the key/value head-size keys (the head size is then hidden / heads)."""
    kv = [("general.architecture", STR, "llama"),
          ("general.alignment", U32, alignment),
          ("llama.block_count", U32, cfg.n_layers),
          ("llama.context_length", U32, ctx_len),
          ("llama.embedding_length", U32, cfg.hidden),
          ("llama.feed_forward_length", U32, cfg.ffn),
          ("llama.attention.head_count", U32, cfg.n_q_heads),
          ("llama.attention.head_count_kv", U32, cfg.n_kv_heads),
          ("llama.rope.freq_base", F32, cfg.rope_theta),
          ("llama.attention.layer_norm_rms_epsilon", F32, cfg.rms_eps),
          ("tokenizer.ggml.tokens", ARR, (STR, [f"tok{i}" for i in range(8)]))]
    if head_keys:
        kv += [("llama.attention.key_length", U32, cfg.head_dim),
               ("llama.attention.value_length", U32, cfg.head_dim)]
    kv += list(extra_kv)

    def mat(name, q, rows, cols):
        return (name, [cols, rows], q.type, np.ascontiguousarray(q.data).tobytes())

    def vec(name, a):
        return (name, [cfg.hidden], 0, np.ascontiguousarray(a, dtype=np.float32).tobytes())

    H, D = cfg.hidden, cfg.head_dim
    QD, KD, F, V = cfg.n_q_heads * D, cfg.n_kv_heads * D, cfg.ffn, cfg.vocab
    ts = [mat("token_embd.weight", w.tok_embd, V, H), vec("output_norm.weight", w.output_norm)]
    if not tied_output:
        ts.append(mat("output.weight", w.output, V, H))
    for i, L in enumerate(w.layers):
        p = f"blk.{i}."
        ts += [vec(p + "attn_norm.weight", L.attn_norm), mat(p + "attn_q.weight", L.wq, QD, H),
               mat(p + "attn_k.weight", L.wk, KD, H), mat(p + "attn_v.weight", L.wv, KD, H),
               mat(p + "attn_output.weight", L.wo, H, QD), vec(p + "ffn_norm.weight", L.ffn_norm),
               mat(p + "ffn_gate.weight", L.w_gate, F, H), mat(p + "ffn_up.weight", L.w_up, F, H),
               mat(p + "ffn_down.weight", L.w_down, H, F)]
    return gguf_bytes(kv, ts, alignment=alignment)
