"""Shared comparison rules for the GPU parity tests.

Tolerances: max |delta logits| <= 1e-4 for the small and medium shapes and
5e-4 for the large one.  Greedy agreement near ties: if the oracle's top-2
margin exceeds 2*tol the GPU's argmax must equal the oracle's; otherwise the
step is an epsilon-tie, both picks are correct, and the GPU's pick must be
within 2*tol of the oracle's maximum (the tolerance alone allows either).
"""
from __future__ import annotations

import numpy as np

TOL = {"small": 1e-4, "medium": 1e-4, "large": 5e-4, "tiny": 1e-4}


def check_argmax(gpu_next, oracle_top1, oracle_top1v, oracle_top2v, gpu_logit_at_pick_oracle, tol):
    """Returns the number of epsilon-ties; raises AssertionError otherwise."""
    ties = 0
    for b in range(len(gpu_next)):
        margin = float(oracle_top1v[b] - oracle_top2v[b])
        if margin > 2 * tol:
            assert int(gpu_next[b]) == int(oracle_top1[b]), (
                f"argmax mismatch in sequence {b}: gpu {int(gpu_next[b])} oracle {int(oracle_top1[b])} "
                f"(margin {margin:.3g})")
        else:
            ties += 1
            if gpu_logit_at_pick_oracle is not None:
                assert gpu_logit_at_pick_oracle[b] >= oracle_top1v[b] - 2 * tol
    return ties


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
