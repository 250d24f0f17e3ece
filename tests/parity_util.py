"""Greedy decode parity between the HIP decode step and the oracle's.

Protocol (logits compared normwise, as elementwise relative error is
ill-posed for logits near 0): per step max|d| <= 5e-3 max|ref| and
||d||_2 <= 5e-3 ||ref||_2.  Both sides decode greedily from the same token
and position.  Where the GPU's token differs from the oracle's and the
oracle's top-2 gap is within 2 max|d| (a near-tie, where either token is
correct to the stated tolerance), the divergence is counted, printed with
its step, and the GPU continues on the oracle's token so later steps still
compare like with like.  A divergence outside a near-tie fails at once, and
more than one near-tie per 16 steps fails the run.

Test infrastructure: it calls the oracle, so only tests use it.
"""
from __future__ import annotations

import numpy as np

LOGIT_TOL = 5e-3


def check_logits(got, ref, what):
    d = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got)), what
    assert d.max() <= LOGIT_TOL * np.abs(ref).max(), f"{what}: max|d| {d.max():.3e} vs {np.abs(ref).max():.3e}"
    assert np.linalg.norm(d) <= LOGIT_TOL * np.linalg.norm(ref), f"{what}: norm"
    return d.max()


def allowed_near_ties(n_steps: int) -> int:
    return n_steps // 16


def greedy_parity_run(model, dec, vocab: int, n_pos: int, first_token: int, n_steps: int, what: str = "",
                      graph: bool = True, oracle_threads: int | None = None, each_step=None, say=None):
    """Decode n_steps tokens on the GPU (`model`, an nt.Model) and in the
    oracle (`dec`, an oracle.Decoder on the same weights and cache), compare
    as the module docstring states, and return a summary dict.  each_step(s,
    logits) sees the GPU logits of every step (for extra checks); say(msg),
    if given, reports each step as it ends."""
    import torch

    from .gpu_util import device, host

    model.set_graph(graph)
    dev = device()
    d_tok = torch.tensor([first_token], dtype=torch.int32, device=dev)
    d_pos = torch.tensor([n_pos], dtype=torch.int32, device=dev)
    logits = torch.empty(vocab, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()          # graphs are only captured on a non-NULL stream
    tok, near, worst = first_token, [], 0.0
    for s in range(n_steps):
        ref, ref_next = dec.step(tok, n_pos + s, nthreads=oracle_threads)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            model.step(d_tok, d_pos, logits, d_tok)  # d_next == d_token: greedy feedback on device
        got = host(logits)
        gpu_next = int(host(d_tok)[0])
        assert int(host(d_pos)[0]) == n_pos + s + 1, f"{what} step {s}: position"
        dmax = check_logits(got, ref, f"{what} step {s}")
        worst = max(worst, dmax / np.abs(ref).max())
        if each_step is not None:
            each_step(s, got)
        if say is not None:
            say(f"{what}: step {s + 1} of {n_steps} compared, max|d| {dmax:.3e}")
        if gpu_next != ref_next:
            top2 = np.sort(ref)[-2:]
            gap = top2[1] - top2[0]
            assert gap <= 2 * dmax, f"{what} step {s}: token {gpu_next} vs oracle {ref_next} (gap {gap:.3e})"
            near.append((s, gpu_next, ref_next, float(gap)))
            print(f"{what}: near-tie at step {s}: GPU {gpu_next}, oracle {ref_next}, top-2 gap {gap:.3e}, "
                  f"max|d| {dmax:.3e}; continuing on the oracle's token", flush=True)
            d_tok.fill_(ref_next)
        tok = ref_next
    torch.cuda.synchronize()
    print(f"{what}: {n_steps} greedy steps from pos {n_pos}, {len(near)} near-ties, "
          f"worst max|d|/max|ref| {worst:.2e}", flush=True)
    assert len(near) <= allowed_near_ties(n_steps), f"{what}: {len(near)} near-ties in {n_steps} steps: {near}"
    return dict(near_ties=len(near), worst=worst, last_token=tok)
