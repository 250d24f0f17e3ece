"""Quantized batch-1 Llama decode for MI355X (gfx950).

The compute path lives in hand-written HIP kernels behind the C-ABI library
``libnt.so`` (declared in ``include/nt.h``); ``block_quantized_decode_dequant_amd.nt``
is the thin ctypes binding over it.  ``synth`` holds the seeded input
generators shared with the tests.
"""
