"""Write the oracle's expected values for the workload parity tests.

    python tests/golden/make_goldens.py [keys...]     (default: every key of STEPS)

Calls only the CPU oracle (oracle/) and the seeded input generator.  For
each workload the oracle runs the prefill, then greedy decoding along its own
argmax tokens.  Stored per workload (tests/golden/wl_<key>.npz):
  tokens      int32 [steps, B]   token fed at decode step k (the oracle's argmax)
  top1, top1v, top2v             per call (prefill + steps) and sequence: argmax,
                                 its logit, the runner-up logit
  sample_idx, sample_logits      full logits of a subset of calls
  kv_pos, kv_k, kv_v             K/V rows of layers 0 and L-1 at a few positions
  weights_check                  fingerprint of the generated weights
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from audio_midi_transformer_amd import synth  # noqa: E402

OUT = os.path.dirname(os.path.abspath(__file__))

# decode steps stored per workload: every run is stored in full (the large
# B=8 run, 8 x 1544 steps of the 48-layer model, takes the oracle about an
# hour or more on 6 threads)
STEPS = {"0": 16, "1": 256, "2": 1544, "3": 512, "3c576": 72, "4": 1544, "4b8": 1544,
         # the W4A8 variant (oracle in its W4A8 mode) of three workloads
         "0a8": 16, "2a8": 1544, "3a8": 512,
         # dense-weight variants (oracle with unquantised, or binary16-rounded,
         # projections); the large one is the pages' half-precision model
         "0f32": 16, "0f16": 16, "2f16": 1544, "4f16": 1544}


def workload_of(key: str):
    """Workload and arithmetic of a golden key: '<workload>' (INT4),
    '<workload>a8' (W4A8), '<workload>f16' or '<workload>f32' (dense)."""
    for suffix in ("a8", "f16", "f32"):
        if key.endswith(suffix):
            return key[:-len(suffix)], suffix
    return key, None


def weights_fingerprint(w: synth.ModelWeights) -> np.ndarray:
    return np.array([float(np.sum(w.tok_emb, dtype=np.float64)),
                     float(np.sum(w.w_qkv[0], dtype=np.float64)),
                     float(np.sum(w.w_down[-1], dtype=np.float64)),
                     float(np.sum(w.lm_head, dtype=np.float64))])


def sample_calls(n_calls: int, batch: int):
    every = 64 if batch == 1 else 128
    idx = set(range(min(9, n_calls)))
    idx |= set(range(0, n_calls, every))
    idx.add(n_calls - 1)
    return np.array(sorted(idx), dtype=np.int32)


def run(key: str) -> None:
    base, mode = workload_of(key)
    wl = synth.WORKLOADS[base]
    steps = STEPS[key]
    t_start = time.time()
    w = synth.model_weights(wl.shape, wl.model_seed)
    m = oracle.OracleModel.from_weights(w, batch=wl.batch, t_cap=wl.t_cap, w4a8=mode == "a8",
                                        dense=mode if mode in ("f16", "f32") else None)
    prefix = synth.workload_prefix(wl) if wl.prefix_len else None
    tokens = synth.workload_tokens(wl) if wl.n_tokens else None
    n_calls = steps + 1
    sidx = sample_calls(n_calls, wl.batch)
    B, V = wl.batch, wl.shape.vocab
    top1 = np.zeros((n_calls, B), np.int32)
    top1v = np.zeros((n_calls, B), np.float32)
    top2v = np.zeros((n_calls, B), np.float32)
    fed = np.zeros((steps, B), np.int32)
    samples = []

    def record(k, logits, nxt):
        srt = np.sort(logits, axis=1)
        top1[k] = nxt
        top1v[k] = logits[np.arange(B), nxt]
        top2v[k] = srt[:, -2]
        if k in set(sidx.tolist()):
            samples.append(logits.copy())

    logits, nxt = m.forward(tokens=tokens, prefix=prefix)
    record(0, logits, nxt)
    print(f"[{key}] prefill done in {time.time() - t_start:.1f}s", flush=True)
    for k in range(1, n_calls):
        fed[k - 1] = nxt
        logits, nxt = m.forward(tokens=nxt.reshape(B, 1))
        record(k, logits, nxt)
        if k % 128 == 0:
            print(f"[{key}] step {k}/{steps} at {time.time() - t_start:.1f}s", flush=True)
    K, Vc = m.kv()
    R0 = wl.prefix_len + wl.n_tokens
    pos = sorted({0, 1, max(0, R0 - 1), R0, R0 + steps // 2, R0 + steps - 1})
    pos = np.array([p for p in pos if p < R0 + steps], dtype=np.int32)
    layers = [0, wl.shape.n_layers - 1]
    kv_k = np.stack([K[l][:, pos] for l in layers]).astype(np.float32)
    kv_v = np.stack([Vc[l][:, pos] for l in layers]).astype(np.float32)
    np.savez_compressed(os.path.join(OUT, f"wl_{key}.npz"), tokens=fed, top1=top1, top1v=top1v,
                        top2v=top2v, sample_idx=sidx, sample_logits=np.stack(samples),
                        kv_pos=pos, kv_layers=np.array(layers, np.int32), kv_k=kv_k, kv_v=kv_v,
                        weights_check=weights_fingerprint(w), position=np.int32(m.position))
    m.close()
    print(f"[{key}] wrote wl_{key}.npz in {time.time() - t_start:.1f}s", flush=True)


if __name__ == "__main__":
    keys = sys.argv[1:] or list(STEPS)
    for k in keys:
        run(k)
