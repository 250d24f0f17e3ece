"""nt_attn_decode_noalloc: decode attention with the library's fixed scratch
array instead of a caller workspace, called through the C ABI (ctypes) and
checked against nt_attn_decode on the same inputs: outputs and both caches
bit for bit (the two share their kernels), on two calls in a row, the second
with a smaller shape; a shape beyond the array is refused before any launch.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_decode_dequant_amd import nt, synth

from .gpu_util import assert_close, device, host, to_dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 8 << 20          # NT_ATTN_NOALLOC_SCRATCH_BYTES in include/nt.h


def _noalloc():
    L = nt.lib()
    fn = L.nt_attn_decode_noalloc
    vp = C.c_void_p
    fn.restype = C.c_int
    fn.argtypes = [C.POINTER(nt.AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp]
    return fn


def _inputs(hq, hkv, d, ctx, pos, seed):
    kc = synth.kv_prefix_bits(seed, 0, 0, hkv, ctx, d, pos)
    vc = synth.kv_prefix_bits(seed, 0, 1, hkv, ctx, d, pos)
    q = synth.normal_f32(seed, 560, hq * d)
    kn = synth.normal_f32(seed, 561, hkv * d)
    vn = synth.normal_f32(seed, 562, hkv * d)
    return q, kn, vn, kc, vc


def _run_both(hq, hkv, d, ctx, pos, theta, seed):
    q, kn, vn, kc, vc = _inputs(hq, hkv, d, ctx, pos, seed)
    desc = nt.attn_desc(hq, hkv, d, ctx, rope_theta=theta)
    dev = device()
    dq, dkn, dvn, dpos = to_dev(q), to_dev(kn), to_dev(vn), torch.tensor([pos], dtype=torch.int32, device=dev)
    # the existing entry point, with a caller workspace
    ws = torch.empty(nt.nt_attn_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    ka, va = to_dev(kc), to_dev(vc)
    oa = torch.empty(hq * d, dtype=torch.float32, device=dev)
    nt.nt_attn_decode(desc, dq, dkn, dvn, ka, va, dpos, oa, ws)
    # the no-allocation entry point, through the C ABI
    kb, vb = to_dev(kc), to_dev(vc)
    ob = torch.full((hq * d,), float("nan"), dtype=torch.float32, device=dev)
    st = _noalloc()(C.byref(desc), C.c_void_p(dq.data_ptr()), C.c_void_p(dkn.data_ptr()),
                    C.c_void_p(dvn.data_ptr()), C.c_void_p(kb.data_ptr()), C.c_void_p(vb.data_ptr()),
                    C.c_void_p(dpos.data_ptr()), C.c_void_p(ob.data_ptr()),
                    C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == nt.NT_OK, nt.lib().nt_last_error().decode(errors="replace")
    got, ref = host(ob), host(oa)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "output differs from nt_attn_decode"
    assert torch.equal(ka, kb) and torch.equal(va, vb), "caches differ from nt_attn_decode"
    return q, kn, vn, kc, vc, got


def test_noalloc_matches_the_workspace_entry_point_twice():
    # first call: the Llama-70B layer shape at full context (2.1 MB of scratch)
    _run_both(64, 8, 128, 4160, 4096, 500000.0, seed=71)
    # second call, smaller: the array keeps the first call's contents
    q, kn, vn, kc, vc, got = _run_both(4, 2, 64, 32, 10, 0.0, seed=72)
    ref = O.attention(q, kn, vn, kc, vc, 4, 2, 64, 32, 10)
    assert_close(got, ref, what="noalloc attention vs oracle")


def test_noalloc_refuses_a_shape_beyond_the_array():
    desc = nt.attn_desc(64, 8, 128, 1 << 17)
    assert nt.nt_attn_workspace_bytes(desc) > SCRATCH_BYTES
    z = C.c_void_p(256)      # never dereferenced: the size check comes first
    st = _noalloc()(C.byref(desc), z, z, z, z, z, z, z, None)
    assert st == nt.NT_ENOMEM
    assert "scratch" in nt.lib().nt_last_error().decode(errors="replace")
