"""Seeded synthetic inputs for the MuScriptor decoder step.

This module only draws numbers and names shapes. It holds none of the
decoder's arithmetic (no quantisation, no normalisation, no attention), so
both the CPU oracle and the HIP path can be fed from it without sharing any
part of the computation.

Shapes follow the pages:
  * widths / heads / depths of the three sizes: MuScriptor model card
    ("Model variants" table) and the Core AI conversion table;
  * MT3 vocabulary of 1393 tokens, greedy decoding: small ONNX conversion
    page, decoder section;
  * prefix of 501 audio frames + 1 dataset slot + K instrument slots: small
    ONNX conversion page, conditioner section (K = 2 here, so P = 504);
  * cache capacity 2504 by default: medium ONNX README, "Quick smoke test".

The conditioner's real output distribution is not on the pages; N(0, 1)
prefix rows stand in for it.  Weights are N(0, 0.02); LayerNorm gains are
1 + N(0, 0.02) and biases N(0, 0.02) so that a dropped or swapped gain or
bias changes the result.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

VOCAB = 1393
HEAD_DIM = 64
GROUP = 32
PREFIX_ROWS = 501 + 1 + 2  # audio frames + dataset slot + two instrument slots


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    d_ff: int
    vocab: int = VOCAB
    head_dim: int = HEAD_DIM
    group: int = GROUP

    @property
    def n_weights(self) -> int:
        """INT4-quantised weights per model (four projections per layer)."""
        d, f = self.d_model, self.d_ff
        return self.n_layers * (3 * d * d + d * d + f * d + d * f)


SMALL = ModelShape("small", 14, 768, 12, 3072)
MEDIUM = ModelShape("medium", 24, 1024, 16, 4096)
LARGE = ModelShape("large", 48, 1536, 24, 6144)


@dataclass(frozen=True)
class Workload:
    """One decoding run: prefill (prefix rows and/or prompt tokens), then
    greedy steps."""
    key: str
    name: str
    shape: ModelShape
    model_seed: int
    batch: int
    prefix_len: int
    n_tokens: int
    decode_steps: int
    t_cap: int
    prefix_seed_base: int = 0
    token_seed: int = 10
    notes: str = ""


WORKLOADS: Dict[str, Workload] = {
    "0": Workload("0", "small decoder, 8 prompt tokens, 16 steps, cache 64",
                  SMALL, 100, 1, 0, 8, 16, 64),
    "1": Workload("1", "small full chunk, prefix 504, 256 steps, cache 1024",
                  SMALL, 100, 1, PREFIX_ROWS, 0, 256, 1024, prefix_seed_base=1000),
    "2": Workload("2", "medium decoder, prefix 504, decode to 2048, cache 2504",
                  MEDIUM, 200, 1, PREFIX_ROWS, 0, 2048 - PREFIX_ROWS, 2504,
                  prefix_seed_base=2000),
    "3": Workload("3", "medium batched B=8, prefix 504, 512 steps, cache 1024",
                  MEDIUM, 200, 8, PREFIX_ROWS, 0, 512, 1024, prefix_seed_base=3000,
                  notes="504 + 512 rows exceed the stated 576-slot cache; the "
                        "capacity is raised to 1024 and the 576 case is run "
                        "separately until the cache is full"),
    "3c576": Workload("3c576", "medium batched B=8, prefix 504, cache 576 (runs until full)",
                      MEDIUM, 200, 8, PREFIX_ROWS, 0, 576 - PREFIX_ROWS, 576,
                      prefix_seed_base=3000),
    "4": Workload("4", "large decoder B=1, prefix 504, decode to 2048, cache 2504",
                  LARGE, 300, 1, PREFIX_ROWS, 0, 2048 - PREFIX_ROWS, 2504,
                  prefix_seed_base=4000),
    "4b8": Workload("4b8", "large decoder B=8, prefix 504, decode to 2048, cache 2504",
                    LARGE, 300, 8, PREFIX_ROWS, 0, 2048 - PREFIX_ROWS, 2504,
                    prefix_seed_base=4000),
}


@dataclass
class ModelWeights:
    """FP32 weights before quantisation. Projection matrices are [N, K]:
    row n is output feature n, K is the input width."""
    shape: ModelShape
    tok_emb: np.ndarray                      # [V, d]
    w_qkv: List[np.ndarray] = field(default_factory=list)   # [3d, d] rows Q | K | V
    w_o: List[np.ndarray] = field(default_factory=list)     # [d, d]
    w_up: List[np.ndarray] = field(default_factory=list)    # [F, d]
    w_down: List[np.ndarray] = field(default_factory=list)  # [d, F]
    ln1_g: List[np.ndarray] = field(default_factory=list)
    ln1_b: List[np.ndarray] = field(default_factory=list)
    ln2_g: List[np.ndarray] = field(default_factory=list)
    ln2_b: List[np.ndarray] = field(default_factory=list)
    lnf_g: np.ndarray = None
    lnf_b: np.ndarray = None
    lm_head: np.ndarray = None               # [V, d]


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def model_weights(shape: ModelShape, seed: int) -> ModelWeights:
    """Draw every tensor from one PCG64 stream in a fixed order: embedding,
    then per layer (Wqkv, Wo, Wup, Wdown, g1, b1, g2, b2), then gf, bf, Wlm."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d, f, v = shape.d_model, shape.d_ff, shape.vocab
    w = ModelWeights(shape=shape, tok_emb=_normal(rng, (v, d), 0.02))
    for _ in range(shape.n_layers):
        w.w_qkv.append(_normal(rng, (3 * d, d), 0.02))
        w.w_o.append(_normal(rng, (d, d), 0.02))
        w.w_up.append(_normal(rng, (f, d), 0.02))
        w.w_down.append(_normal(rng, (d, f), 0.02))
        w.ln1_g.append(np.float32(1.0) + _normal(rng, (d,), 0.02))
        w.ln1_b.append(_normal(rng, (d,), 0.02))
        w.ln2_g.append(np.float32(1.0) + _normal(rng, (d,), 0.02))
        w.ln2_b.append(_normal(rng, (d,), 0.02))
    w.lnf_g = np.float32(1.0) + _normal(rng, (d,), 0.02)
    w.lnf_b = _normal(rng, (d,), 0.02)
    w.lm_head = _normal(rng, (v, d), 0.02)
    return w


def prefix_rows(shape: ModelShape, seed: int, rows: int) -> np.ndarray:
    """One sequence's conditioner prefix stand-in, N(0,1) float32 [rows, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(size=(rows, shape.d_model), dtype=np.float32)


def workload_prefix(wl: Workload, batch: int | None = None) -> np.ndarray:
    """[B, P, d]; sequence b uses seed prefix_seed_base + b, so every sequence
    (and so its instrument-slot rows) differs."""
    b_n = wl.batch if batch is None else batch
    if wl.prefix_len == 0:
        return np.zeros((b_n, 0, wl.shape.d_model), dtype=np.float32)
    return np.stack([prefix_rows(wl.shape, wl.prefix_seed_base + b, wl.prefix_len)
                     for b in range(b_n)])


def cfg_pair_prefix(wl: Workload, pairs: int | None = None, class_rows: int = 2) -> np.ndarray:
    """Prefixes of conditional/unconditional pairs, [2 Np, P, d]: rows
    0 .. Np-1 are workload_prefix; partner Np + i repeats row i's prefix and
    redraws its last `class_rows` rows (the conditioner's prefix ends with
    its class rows) from seed prefix_seed_base + 10000 + i."""
    n = wl.batch if pairs is None else pairs
    cond = workload_prefix(wl, n)
    uncond = cond.copy()
    k = min(class_rows, wl.prefix_len)
    for i in range(n):
        if k:
            uncond[i, -k:] = prefix_rows(wl.shape, wl.prefix_seed_base + 10000 + i, k)
    return np.concatenate([cond, uncond])


def workload_tokens(wl: Workload, batch: int | None = None) -> np.ndarray:
    """Prompt token ids [B, S] (int64), uniform over the vocabulary."""
    b_n = wl.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(wl.token_seed))
    return rng.integers(0, wl.shape.vocab, size=(b_n, wl.n_tokens), dtype=np.int64)


def random_matrix(seed: int, n: int, k: int, scale: float = 0.02) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal(rng, (n, k), scale)


def tiny_shape(n_layers=2, d_model=128, n_heads=2, d_ff=512, vocab=97) -> ModelShape:
    """Small shapes for tests the oracle finishes in well under a second."""
    return ModelShape("tiny", n_layers, d_model, n_heads, d_ff, vocab)


def tie_head_rows(w: ModelWeights, rows, seed: int = 0, bias_norm: float = 40.0, gain: float = 4.0) -> ModelWeights:
    """Inputs with an exact greedy tie at every position.

    The final LayerNorm bias is replaced by a long random direction u
    (|bias| = bias_norm) and every LM-head row listed in `rows` by the same
    vector gain * u / |u|.  Those rows then produce bit-equal logits (same
    row, same input, same arithmetic), near gain * bias_norm, far above every
    other logit (a random row of N(0, 0.02) entries gives about +-1).
    Modifies w in place and returns it."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.standard_normal(w.shape.d_model)
    u /= np.sqrt(np.sum(u * u))
    w.lnf_b = (bias_norm * u).astype(np.float32)
    row = (gain * u).astype(np.float32)
    for r in rows:
        w.lm_head[r] = row
    return w
