"""GPU parity for the block decoders, the device encoder and the fused
dequantize-GEMV, against the fp64 oracle on the same seeded inputs.

Bars: decoded values and encoded blocks bit-exact; GEMV within
1e-4 + 2e-3 |y| elementwise.  Shapes span one block, several slices of a
workgroup, ragged row tiles, two units per lane (cols > 32768), and the full
Q8_0 4096 x 4096 and K-quant 70B projection sweep in the launch configuration
the benchmark times.
"""
import glob
import os

import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_decode_dequant_amd import nt, synth, workloads

from .gpu_util import assert_close, device, host, to_dev
from .test_oracle_formats import load_golden

pytestmark = pytest.mark.gpu

TYPES = [O.Q8_0, O.Q4_0, O.Q4_K, O.Q5_K, O.Q6_K]
TID = ["q8_0", "q4_0", "q4_k", "q5_k", "q6_k"]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blocks(t, nvals, seed, std=0.02):
    return O.quantize(t, synth.normal_f32(seed, 300 + t, nvals, std=std))


# ---- dequant -------------------------------------------------------------------
@pytest.mark.parametrize("t", TYPES, ids=TID)
def test_dequant_bit_exact(t):
    """Both kernels: a 16-byte-aligned output (256-value windows, one 16-byte
    store per lane) and a 4-byte-aligned one (one value per thread); for the
    32-value formats the last window is partial (3 blocks past a multiple of 8)."""
    device()
    parts = [_blocks(t, 64 * 256, 1), _blocks(t, 8 * 256, 2, std=3.0)]
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.txt"))):
        gt, blk, _ = load_golden(path)
        if gt == t:
            parts.append(blk)
    blocks = np.concatenate(parts)
    nb = blocks.size // O.block_bytes(t)
    if O.block_elems(t) == 32:
        extra = (8 - nb % 8 + 3) % 8 or 8          # leaves 3 blocks in the last window
        blocks = np.concatenate([blocks, _blocks(t, 32 * extra, 3)])
        assert (blocks.size // O.block_bytes(t)) % 8 == 3
    n = blocks.size // O.block_bytes(t) * O.block_elems(t)
    ref = O.dequant(t, blocks, n)
    dev_blocks = to_dev(blocks)
    out = torch.full((n + 8,), float("nan"), dtype=torch.float32, device=device())
    for off in (0, 1):
        nt.nt_dequant(t, dev_blocks, out[off:off + n], n)
        got = host(out)
        assert np.array_equal(got[off:off + n].view(np.uint32), ref.view(np.uint32)), f"output offset {4 * off} bytes"
        assert np.isnan(got[off + n:]).all(), "written past n"


def test_dequant_q8_0_subnormal_scales():
    """The Q8_0 GEMV recipe has fp16-subnormal scales in ~0.5% of blocks."""
    W = synth.q8_0_random_matrix(0, 256, 4096)
    d = synth.q8_0_random_parts(0, 256, 4096)[0]
    assert np.count_nonzero((d & 0x7C00) == 0) > 50
    n = 256 * 4096
    out = torch.empty(n, dtype=torch.float32, device=device())
    nt.nt_dequant_q8_0(to_dev(W), out, n)
    assert np.array_equal(host(out).view(np.uint32), O.dequant(O.Q8_0, W, n).view(np.uint32))


# ---- device encoder ---------------------------------------------------------------
@pytest.mark.parametrize("t", TYPES, ids=TID)
def test_quantize_bit_exact(t):
    x = np.concatenate([synth.normal_f32(4, 310 + t, 128 * 256, std=0.02),
                        synth.normal_f32(4, 320 + t, 16 * 256, std=1.0),
                        np.zeros(256, np.float32),
                        np.linspace(-1, 3, 512).astype(np.float32),
                        synth.normal_f32(4, 330 + t, 256, std=1e-6)])
    be = O.block_elems(t)
    blocks = torch.zeros(x.size // be * O.block_bytes(t), dtype=torch.uint8, device=device())
    nt.nt_quantize(t, to_dev(x), blocks, x.size)
    assert np.array_equal(host(blocks), O.quantize(t, x))


# ---- GEMV ----------------------------------------------------------------------------
def _gemv_case(t, rows, cols, seed, accumulate=False):
    W = _blocks(t, rows * cols, seed)
    x = synth.normal_f32(seed, 400 + t, cols)
    y0 = synth.normal_f32(seed, 410 + t, rows) if accumulate else np.zeros(rows, np.float32)
    dy = torch.empty(rows + 64, dtype=torch.float32, device=device())
    dy.fill_(12345.0)
    dy[:rows] = to_dev(y0)
    nt.nt_gemv(t, to_dev(W), to_dev(x), dy, rows, cols, accumulate)
    got = host(dy)
    assert np.all(got[rows:] == 12345.0), "rows past the end were written"
    ref = O.gemv(t, W, rows, cols, x) + (y0.astype(np.float64) if accumulate else 0.0)
    assert_close(got[:rows], ref, what=f"gemv {TID[TYPES.index(t)]} {rows}x{cols}")


# ... plus one row on the fast path, two rows of the 28672-column (per-wave
# staging) layout, and the largest column count the calls accept
SHAPES = [(1, 256), (3, 512), (37, 1024), (101, 4352), (64, 40960), (5, 2048 + 256),
          (1, 8192), (2, 28672), (3, 65536)]


@pytest.mark.parametrize("t", TYPES, ids=TID)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_gemv_parity(t, rows, cols):
    _gemv_case(t, rows, cols, seed=rows + cols)


@pytest.mark.parametrize("t", TYPES, ids=TID)
def test_gemv_accumulate(t):
    _gemv_case(t, 77, 3072, seed=9, accumulate=True)


@pytest.mark.parametrize("t", [O.Q8_0, O.Q4_0], ids=["q8_0", "q4_0"])
def test_gemv_odd_block_count_and_single_block_rows(t):
    # 33 blocks per row: rows start at odd block indices and 2-byte offsets
    _gemv_case(t, 19, 33 * 32, seed=3)
    _gemv_case(t, 7, 32, seed=4)


def test_gemv_q8_0_workload_full():
    """The 4096 x 4096 Q8_0 GEMV workload, every row against the oracle."""
    wl = workloads.Q8_0_GEMV
    rows, cols = wl["rows"], wl["cols"]
    W = synth.q8_0_random_matrix(workloads.SEED, rows, cols)
    x = synth.activation(workloads.SEED, synth.Q8_CFG_X, cols)
    dy = torch.empty(rows, dtype=torch.float32, device=device())
    nt.nt_gemv_q8_0(to_dev(W), to_dev(x), dy, rows, cols)
    assert_close(host(dy), O.gemv(O.Q8_0, W, rows, cols, x), what="q8_0 4096x4096")


@pytest.mark.parametrize("si", range(len(workloads.KQ_SHAPES)))
def test_gemv_kquant_sweep_full(si):
    """The 70B projection shapes in Q4_K and Q6_K: device-encoded blocks equal
    the oracle's, and every output row is within tolerance."""
    rows, cols = workloads.KQ_SHAPES[si]
    w = synth.normal_f32(workloads.SEED, workloads.kq_w_stream(si), rows * cols, std=0.02)
    x = synth.activation(workloads.SEED, workloads.kq_x_stream(si), cols)
    dw, dx = to_dev(w), to_dev(x)
    for t in (O.Q4_K, O.Q6_K):
        ref_blocks = O.quantize(t, w)
        blocks = torch.empty(ref_blocks.size, dtype=torch.uint8, device=device())
        nt.nt_quantize(t, dw, blocks, rows * cols)
        assert np.array_equal(host(blocks), ref_blocks), "device encoder differs from the oracle"
        dy = torch.empty(rows, dtype=torch.float32, device=device())
        nt.nt_gemv(t, blocks, dx, dy, rows, cols)
        assert_close(host(dy), O.gemv(t, ref_blocks, rows, cols, x), what=f"{t} {rows}x{cols}")
        del blocks


@pytest.mark.parametrize("t", TYPES, ids=TID)
def test_gemv_deterministic(t):
    rows, cols = 512, 8192
    W = to_dev(_blocks(t, rows * cols, 11))
    x = to_dev(synth.normal_f32(11, 420, cols))
    a = torch.empty(rows, dtype=torch.float32, device=device())
    b = torch.empty(rows, dtype=torch.float32, device=device())
    nt.nt_gemv(t, W, x, a, rows, cols)
    nt.nt_gemv(t, W, x, b, rows, cols)
    assert torch.equal(a, b)


def test_gemv_zero_rows_is_a_no_op():
    dev = device()
    W = torch.zeros(144, dtype=torch.uint8, device=dev)
    x = torch.zeros(256, dtype=torch.float32, device=dev)
    y = torch.full((4,), 7.0, device=dev)
    nt.nt_gemv_q4_k(W, x, y, 0, 256)
    assert torch.all(y == 7.0)


# ---- LDS-ring path: 4-byte copies (rows only word-aligned), many rows per workgroup ----
VEC4_CASES = [(O.Q8_0, 9, 320), (O.Q8_0, 20000, 320), (O.Q8_0, 130, 2112), (O.Q4_0, 20000, 320),
              (O.Q4_0, 130, 2112), (O.Q6_K, 70, 1536), (O.Q6_K, 12000, 1536), (O.Q6_K, 33, 6144)]


@pytest.mark.parametrize("t,rows,cols", VEC4_CASES,
                         ids=[f"{TID[TYPES.index(t)]}-{r}x{c}" for t, r, c in VEC4_CASES])
def test_gemv_word_aligned_rows_and_deep_ring(t, rows, cols):
    info = nt.nt_gemv_launch_info(t, rows, cols)
    assert info["fast"], info
    _gemv_case(t, rows, cols, seed=rows + 7 * cols)


# ---- fused variants: several matrices, RMSNorm prologue, SwiGLU epilogue ---------------
# 2048 / 4096 columns: one column slice (shared activation area, row groups);
# 8192: two slices (shared area with RMSNorm, per-wave staging without);
# 2112 / 1536: rows only word-aligned (4-byte copies, per-wave staging)
FUSED_COLS = {O.Q8_0: [2048, 2112], O.Q4_0: [2048, 2112], O.Q4_K: [2048, 4096, 8192], O.Q5_K: [2048, 8192],
              O.Q6_K: [2048, 1536, 8192]}


def _norm_inputs(cols, seed):
    x = synth.normal_f32(seed, 430, cols, std=3.0)
    g = (1.0 + synth.normal_f32(seed, 431, cols, std=0.1)).astype(np.float32)
    return x, g


@pytest.mark.parametrize("t", TYPES, ids=TID)
@pytest.mark.parametrize("norm", [True, False], ids=["norm", "plain"])
def test_gemv_multi_parity(t, norm):
    eps = 1e-5
    for cols in FUSED_COLS[t]:
        rows = [37, 5, 64]
        Ws = [_blocks(t, r * cols, 50 + i) for i, r in enumerate(rows)]
        x, g = _norm_inputs(cols, cols)
        n = O.rmsnorm(x, g, eps) if norm else x.astype(np.float64)
        y0 = [synth.normal_f32(cols, 440 + i, r) for i, r in enumerate(rows)]
        acc = not norm                     # the plain variant also checks accumulate
        ys = [to_dev(y) if acc else torch.full((r,), 9.0, device=device()) for y, r in zip(y0, rows)]
        nt.nt_gemv_multi(t, [to_dev(W) for W in Ws], rows, ys, cols, to_dev(x), to_dev(g) if norm else None,
                         eps, accumulate=acc)
        for i, (W, r) in enumerate(zip(Ws, rows)):
            ref = O.gemv(t, W, r, cols, n) + (y0[i].astype(np.float64) if acc else 0.0)
            assert_close(host(ys[i]), ref, what=f"multi {TID[TYPES.index(t)]} seg {i} cols {cols}")


@pytest.mark.parametrize("t", TYPES, ids=TID)
def test_gemv_swiglu_parity(t):
    eps = 1e-5
    for cols in FUSED_COLS[t]:
        rows = 301
        Wg, Wu = _blocks(t, rows * cols, 60), _blocks(t, rows * cols, 61)
        x, g = _norm_inputs(cols, cols + 1)
        n = O.rmsnorm(x, g, eps)
        h = torch.full((rows + 8,), 5.0, device=device())
        nt.nt_gemv_swiglu(t, to_dev(Wg), to_dev(Wu), rows, cols, to_dev(x), h, gain=to_dev(g), eps=eps)
        got = host(h)
        assert np.all(got[rows:] == 5.0)
        ref = O.swiglu(O.gemv(t, Wg, rows, cols, n), O.gemv(t, Wu, rows, cols, n))
        assert_close(got[:rows], ref, what=f"swiglu {TID[TYPES.index(t)]} cols {cols}")


# Shared-area layout at sizes where the row groups refill their rings (more rows per
# wave than ring stages), where most row groups have no row at all, and for rows
# wider than two column slices.
SHARED_CASES = [(O.Q8_0, 7500, 4096, False), (O.Q8_0, 3, 4096, True), (O.Q4_0, 9000, 2048, True),
                (O.Q4_K, 5000, 8192, True), (O.Q6_K, 7, 8192, True), (O.Q6_K, 10500, 4096, False),
                # wider rows whose activation area still fits beside one row group
                (O.Q8_0, 600, 14336, False), (O.Q4_K, 300, 16384, True), (O.Q6_K, 200, 12288, False),
                (O.Q5_K, 5000, 8192, True), (O.Q5_K, 9, 4096, False), (O.Q5_K, 250, 12288, True)]


@pytest.mark.parametrize("t,rows,cols,norm", SHARED_CASES,
                         ids=[f"{TID[TYPES.index(t)]}-{r}x{c}-{'norm' if n else 'plain'}" for t, r, c, n in SHARED_CASES])
def test_gemv_shared_activation_layout(t, rows, cols, norm):
    eps = 1e-5
    W = _blocks(t, rows * cols, 70 + rows)
    x, g = _norm_inputs(cols, rows + cols)
    n = O.rmsnorm(x, g, eps) if norm else x.astype(np.float64)
    y = torch.full((rows,), 3.0, device=device())
    nt.nt_gemv_multi(t, [to_dev(W)], [rows], [y], cols, to_dev(x), to_dev(g) if norm else None, eps)
    assert_close(host(y), O.gemv(t, W, rows, cols, n), what=f"shared {TID[TYPES.index(t)]} {rows}x{cols}")


def test_fused_gemv_rejects_shapes_outside_the_fast_path():
    dev = device()
    W = torch.zeros(210 * 4, dtype=torch.uint8, device=dev)
    x = torch.zeros(256, dtype=torch.float32, device=dev)
    y = torch.zeros(4, dtype=torch.float32, device=dev)
    with pytest.raises(nt.NTError) as e:
        nt.nt_gemv_multi(O.Q6_K, [W], [4], [y], 256, x)       # 210-byte rows: not word-aligned
    assert e.value.status == nt.NT_ESHAPE


def test_gemv_from_several_threads():
    """Calls are thread-safe: four host threads, each on its own stream, launch
    GEMVs of different formats and shapes (first launches included, so the
    per-device launch settings are filled concurrently); every result equals
    the same launch made alone."""
    import threading
    dev = device()
    cases = [(O.Q4_K, 300, 8192), (O.Q6_K, 200, 28672), (O.Q5_K, 257, 4096), (O.Q8_0, 129, 14336)]
    inputs = []
    for i, (t, rows, cols) in enumerate(cases):
        W = to_dev(_blocks(t, rows * cols, 80 + i))
        x = to_dev(synth.normal_f32(80 + i, 450, cols))
        inputs.append((t, rows, cols, W, x))
    outs = [torch.empty(rows, dtype=torch.float32, device=dev) for _, rows, *_ in inputs]
    torch.cuda.synchronize()            # inputs in place before other streams read them
    errors = []

    def work(k):
        try:
            t, rows, cols, W, x = inputs[k]
            s = torch.cuda.Stream()
            for _ in range(20):
                nt.nt_gemv(t, W, x, outs[k], rows, cols, stream=s)
            s.synchronize()
        except Exception as e:          # noqa: BLE001 - reported below
            errors.append(e)

    ths = [threading.Thread(target=work, args=(k,)) for k in range(len(inputs))]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    assert not errors, errors
    for k, (t, rows, cols, W, x) in enumerate(inputs):
        ref = torch.empty(rows, dtype=torch.float32, device=dev)
        nt.nt_gemv(t, W, x, ref, rows, cols)
        torch.cuda.synchronize()
        assert torch.equal(outs[k], ref), f"case {k}"
