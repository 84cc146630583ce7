"""Shared comparison rules for the GPU parity tests.

Tolerances: max |delta logits| <= 1e-4 for the small and medium shapes and
5e-4 for the large one.  Greedy agreement near ties: if the oracle's top-2
margin exceeds 2*tol the GPU's argmax must equal the oracle's; otherwise the
step is an epsilon-tie, both picks are correct, and the GPU's pick must be
within 2*tol of the oracle's maximum (the tolerance alone allows either).
Independently of the oracle, the GPU's pick must be exactly the argmax of
the GPU's own logits with the lowest index winning among bit-equal maxima
(the tie rule of greedy decoding), at every step.
"""
from __future__ import annotations

import numpy as np

TOL = {"small": 1e-4, "medium": 1e-4, "large": 5e-4, "tiny": 1e-4}


def check_own_argmax(gpu_next, gpu_logits, what: str = ""):
    """gpu_next [B] must equal np.argmax(gpu_logits, axis=1): the first index
    of the maximum, so an exact tie goes to the lowest index."""
    gpu_next = np.asarray(gpu_next).reshape(-1)
    gpu_logits = np.asarray(gpu_logits).reshape(len(gpu_next), -1)
    want = np.argmax(gpu_logits, axis=1)
    bad = np.nonzero(gpu_next != want)[0]
    assert len(bad) == 0, (f"{what}: pick is not the argmax of the GPU's own logits in sequence {int(bad[0])}: "
                           f"{int(gpu_next[bad[0]])} vs {int(want[bad[0]])}")


def check_argmax(gpu_next, oracle_top1, oracle_top1v, oracle_top2v, oracle_logit_at_gpu_pick, tol):
    """Returns the number of epsilon-ties; raises AssertionError otherwise.
    oracle_logit_at_gpu_pick: the oracle's logit at the GPU's pick, or None."""
    ties = 0
    for b in range(len(gpu_next)):
        margin = float(oracle_top1v[b] - oracle_top2v[b])
        if margin > 2 * tol:
            assert int(gpu_next[b]) == int(oracle_top1[b]), (
                f"argmax mismatch in sequence {b}: gpu {int(gpu_next[b])} oracle {int(oracle_top1[b])} "
                f"(margin {margin:.3g})")
        else:
            ties += 1
            if oracle_logit_at_gpu_pick is not None:
                assert oracle_logit_at_gpu_pick[b] >= oracle_top1v[b] - 2 * tol
    return ties


def check_greedy(gpu_next, gpu_logits, oracle_logits, tol, what: str = ""):
    """Both greedy checks of one call: the GPU's pick is the exact argmax of
    its own logits, and it agrees with the oracle's outside epsilon-ties (at
    an epsilon-tie the oracle's logit at the GPU's pick is within 2*tol of
    the oracle's maximum).  Returns the number of epsilon-ties."""
    gpu_next = np.asarray(gpu_next).reshape(-1)
    oracle_logits = np.asarray(oracle_logits).reshape(len(gpu_next), -1)
    check_own_argmax(gpu_next, gpu_logits, what)
    at_pick = oracle_logits[np.arange(len(gpu_next)), gpu_next]
    return check_argmax(gpu_next, *top2(oracle_logits), at_pick, tol)


def compare_logits(gpu_logits: np.ndarray, oracle_logits: np.ndarray, tol: float, what: str):
    d = np.abs(gpu_logits.astype(np.float64) - oracle_logits.astype(np.float64))
    worst = float(np.nanmax(d)) if d.size else 0.0
    assert np.all(np.isfinite(gpu_logits)), f"{what}: non-finite GPU logits"
    assert worst <= tol, f"{what}: max |delta| {worst:.3g} > {tol}"
    return worst


def top2(logits: np.ndarray):
    nxt = np.argmax(logits, axis=1)
    srt = np.sort(logits, axis=1)
    return nxt, logits[np.arange(len(nxt)), nxt], srt[:, -2]
