"""Benchmark of the MuScriptor INT4 decoder step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--path auto]

One bench step is one whole pass of the hot path over one batch: the prefill
of the workload's prefix / prompt rows followed by every greedy decode step
of the workload (for the medium workload: 504 prefix rows, then decoding
until the cache holds 2048 positions).  Inputs are seeded synthetic tensors
already resident in GPU memory; decoding feeds the device argmax back without
returning to the host.

Printed (one JSON line): steady-state decode ms/token (steps 8 onward) as
`value`, tokens/s, achieved HBM GB/s from algorithmic bytes, prefill time and
MFMA utilisation, a roofline object for the decode launch, and the CPU
oracle timed on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode ms/token + achieved HBM GB/s, medium W4g32 decoder, cache 2504, B=1"
HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
INT8_MFMA_PEAK_TOPS = 5000.0
# INT4 projections of W4A32 models run on BF16 MFMA with every activation
# split into three bf16 pieces: three BF16 products per FP32 product, so the
# matrix-core ceiling of that form is a third of the dense BF16 peak
BF16X3_MFMA_PEAK_TFLOPS = 2500.0 / 3
STEADY_FROM = 8


# bytes per projection weight: INT4 nibble + FP32 scale per 32; binary16; binary32
WEIGHT_BYTES = {"int4": 0.5 + 4.0 / 32, "f16": 2.0, "f32": 4.0}


def step_bytes(shape, B: int, T: int, wbytes: float = WEIGHT_BYTES["int4"]) -> float:
    """Algorithmic HBM bytes of one decode step over B sequences with T keys
    (the new row included): the four projections' weights (packed INT4
    nibbles + FP32 group scales, or dense values), FP32 LM head, LayerNorm
    parameters, live K/V read, new K/V row written, embedding row, logits,
    token in / argmax out."""
    L, d, F, V = shape.n_layers, shape.d_model, shape.d_ff, shape.vocab
    w_per_layer = 3 * d * d + d * d + 2 * d * F
    weights = wbytes * w_per_layer * L + 4.0 * V * d + 4.0 * (4 * L * d + 2 * d)
    per_seq = 8.0 * L * d * T + 8.0 * L * d + 4.0 * d + 4.0 * V + 16.0
    return weights + B * per_seq


def prefill_flops(shape, B: int, M: int) -> float:
    L, d, F, V = shape.n_layers, shape.d_model, shape.d_ff, shape.vocab
    w_per_layer = 3 * d * d + d * d + 2 * d * F
    return B * (2.0 * M * w_per_layer * L + 2.0 * L * d * M * (M + 1) + 2.0 * d * V)


# sources that build and launch each profiled kernel (its traffic record is
# void once any of them changes)
KERNEL_SOURCES = {"mt_decode_step_persistent": ("mt_decode_persistent.hip", "mt_pd_common.h", "mt_internal.h",
                                                  "mt_api.cpp"),
                  "mt_decode_step_batched": ("mt_decode_batched.hip", "mt_pd_common.h", "mt_internal.h",
                                             "mt_api.cpp")}


def kernel_source_hash(kernel: str = "mt_decode_step_persistent") -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "audio_midi_transformer_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel) or sorted(os.listdir(csrc))
    for name in names:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload_key: str, variant: str = ""):
    """HBM traffic per launch from committed rocprofv3 counter summaries, or
    None when they are missing or were taken on different kernel sources.
    `variant` is "" (INT4 weights, FP32 activations), "a8", "f16" or "f32"."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_wl{workload_key}{variant}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, weights, prefix_np, tokens_np, max_steps: int = 8, w4a8: bool = False,
                 dense=None, cfg=None):
    """The CPU oracle as it stands, on this host, on a bounded sample of the
    workload: its prefill, then `max_steps` greedy decode steps (with `cfg`,
    of the 2B pair rows, each followed by the oracle's guidance)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    os.environ["OMP_NUM_THREADS"] = str(cores)
    rows = wl.batch * (2 if cfg is not None else 1)
    m = oracle.OracleModel.from_weights(weights, batch=rows, t_cap=wl.t_cap, w4a8=w4a8, dense=dense)

    def pick(lg, nxt):
        return np.concatenate([oracle.cfg_combine(lg, cfg)[1]] * 2) if cfg is not None else nxt

    t0 = time.perf_counter()
    nxt = pick(*m.forward(tokens=tokens_np, prefix=prefix_np))
    t1 = time.perf_counter()
    n = min(max_steps, wl.decode_steps)
    for _ in range(n):
        nxt = pick(*m.forward(tokens=nxt.reshape(rows, 1)))
    t2 = time.perf_counter()
    m.close()
    return {
        "value": (t2 - t1) * 1000.0 / n,
        "unit": "ms/token",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"oracle prefill of {wl.prefix_len + wl.n_tokens} rows "
                   f"({(t1 - t0) * 1000.0:.0f} ms) then {n} greedy decode steps of the same "
                   f"workload, B={rows}{' (CFG pairs)' if cfg is not None else ''}; "
                   f"value = mean ms per decode step"),
        "prefill_ms": (t1 - t0) * 1000.0,
    }


KERNEL_SYMBOLS = {"mt_decode_step_persistent": "k_decode_step<", "mt_decode_step_batched": "k_decode_xcd<"}


def reduce_counters(fetch_csv: str, write_csv: str, workload_key: str, calib_mib: int,
                    commands: list) -> dict:
    """HBM bytes per launch of the single-launch decode step (the persistent
    step at one sequence, the batched step at 3 to 8) from two rocprofv3
    `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` counter files of one bench pass
    (steps 1, warmup 0, with the calibration copy).  Each counter is scaled by
    the bytes a plain device copy of `calib_mib` MiB really moves over what
    that counter read for it (the largest copy dispatched before the
    library's first kernel), then
    averaged over the launches the bench's steady window covers."""
    import csv

    from audio_midi_transformer_amd import synth

    kernel = "mt_decode_step_persistent" if synth.WORKLOADS[workload_key].batch <= 2 else "mt_decode_step_batched"

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        first_mt = min(int(r["Dispatch_Id"]) for r in rows if "mt::" in r["Kernel_Name"])
        # the calibration copy runs before any of the library's kernels
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and int(r["Dispatch_Id"]) < first_mt]
        kern = [float(r["Counter_Value"]) for r in rows
                if KERNEL_SYMBOLS[kernel] in r["Kernel_Name"]]
        return max(copies), kern

    known_kib = float(calib_mib) * 1024.0
    f_copy, f_kern = load(fetch_csv, "FETCH_SIZE")
    w_copy, w_kern = load(write_csv, "WRITE_SIZE")
    f_scale, w_scale = known_kib / f_copy, known_kib / w_copy
    # the pass's steady window (launches past it: the bench's point near the
    # end of the cache)
    n_dec = synth.WORKLOADS[workload_key].decode_steps
    f_kern, w_kern = f_kern[STEADY_FROM:n_dec], w_kern[STEADY_FROM:n_dec]
    fetch = float(np.mean(f_kern)) * 1024.0 * f_scale
    write = float(np.mean(w_kern)) * 1024.0 * w_scale
    return {
        "kernel": kernel,
        "workload": workload_key,
        "source_hash": kernel_source_hash(kernel),
        "launches": len(f_kern),
        "calibration_copy_bytes": int(known_kib * 1024),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "fetch_bytes_per_launch": round(fetch, 1),
        "write_bytes_per_launch": round(write, 1),
        "bytes_per_launch": round(fetch + write, 1),
        "commands": commands,
    }


def phase_summary(trace: np.ndarray, T: int, wl) -> dict:
    """Median phase durations (us) over layers 1 .. L-2 of one persistent
    step from its wall-clock stamps [256 workgroups, L + 1, 24 slots] (100 MHz
    ticks).  Slots per layer: 0 phase start, 1 previous FFN-down output
    gathered, 2 LN1 done, 15 q_h done, 3 K/V chunk in LDS, 12 scores,
    13 softmax sums, 14 weighted V sum, 4 partial done, 5 partials gathered
    (head leader), 17 merged head published, 18 K/V rows done (workgroups
    without attention duty), 6 attention output gathered, 7 O rows
    published, 8 O output gathered, 9 FFN-up published, 10 FFN-up output
    gathered, 11 FFN-down published."""
    tr = trace.astype(np.int64)
    L = tr.shape[1] - 1
    lay = tr[:, 1:L - 1, :]
    us = 0.01

    def med(mask, a, b):
        return round(float(np.median((lay[mask, :, b] - lay[mask, :, a]) * us)), 3)

    leader = tr[:, 1, 5] != 0
    free = (tr[:, 1, 18] != 0) & (tr[:, 1, 6] != 0)
    per_layer = (tr[:, 2:L, 0] - tr[:, 1:L - 1, 0]) * us
    lead = {"f_exchange_wait": med(leader, 0, 1), "ln1": med(leader, 1, 2), "q_h": med(leader, 2, 15),
            "chunk_wait": med(leader, 15, 3), "scores": med(leader, 3, 12), "softmax": med(leader, 12, 13),
            "weighted_v": med(leader, 13, 14), "partial_out": med(leader, 14, 4),
            "partials_gather": med(leader, 4, 5), "merge_publish": med(leader, 5, 17),
            "o_exchange_wait": med(leader, 17, 8), "ln2_up_publish": med(leader, 8, 9),
            "u_exchange_wait": med(leader, 9, 10), "down_publish": med(leader, 10, 11)}
    fr = {"f_exchange_wait": med(free, 0, 1), "ln1": med(free, 1, 2), "kv_rows": med(free, 2, 18),
          "attention_wait": med(free, 18, 6), "o_rows_publish": med(free, 6, 7),
          "o_exchange_wait": med(free, 7, 8), "ln2_up_publish": med(free, 8, 9),
          "u_exchange_wait": med(free, 9, 10), "down_publish": med(free, 10, 11)}
    return {"workload": wl.key, "keys": T, "layers": L, "layer_us_median": round(float(np.median(per_layer)), 3),
            "head_leader_us": lead, "free_workgroup_us": fr,
            "workgroups": {"head_leaders": int(leader.sum()), "free": int(free.sum())}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="2")
    ap.add_argument("--path", choices=["auto", "kernels", "persistent", "batched"], default="auto")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="override the number of decode steps per pass (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--w4a8", action="store_true",
                    help="the W4A8 variant: INT8 activation codes per row and group of 32, INT32 group sums")
    ap.add_argument("--weights", choices=["int4", "f16", "f32"], default="int4",
                    help="projection weights: INT4 group-32 (default) or the dense binary16 / binary32 variants")
    ap.add_argument("--batch", type=int, default=None,
                    help="run the workload with this many sequences instead of its own batch "
                         "(each with its own seeded prefix)")
    ap.add_argument("--cfg", type=float, default=None, metavar="COEF",
                    help="classifier-free guidance: each of the workload's sequences becomes a "
                         "conditional/unconditional pair (2B rows), the guided argmax is fed to both")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the bench, copy a buffer of this many MiB device-to-device three "
                         "times (a plain copy of known size, to scale HBM byte counters)")
    ap.add_argument("--reduce-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="reduce two rocprofv3 counter files of a --calibration-copy-mib run to the "
                         "per-launch HBM traffic record (printed as JSON) and exit")
    ap.add_argument("--phase-trace", type=int, default=None, metavar="T",
                    help="persistent step only: prefill the workload, decode greedily until the cache "
                         "holds T positions with per-phase wall-clock stamps (MT_TRACE=1), print the "
                         "median phase durations of the last step's layers as JSON and exit")
    args = ap.parse_args()
    if args.w4a8 and args.weights != "int4":
        ap.error("--w4a8 needs --weights int4")
    variant = "a8" if args.w4a8 else "" if args.weights == "int4" else args.weights
    if args.reduce_counters:
        cmds = [f"rocprofv3 --pmc {c} -f csv -d <dir> -o pmc -- python3 bench.py --workload {args.workload} "
                f"--steps 1 --warmup 0 --no-cpu-baseline --calibration-copy-mib {args.calibration_copy_mib}"
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
        print(json.dumps(reduce_counters(*args.reduce_counters, args.workload, args.calibration_copy_mib, cmds),
                         indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decoder step's natural shard is independent "
              "sequences (no collective), so N GPUs run N copies of this bench; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch
    from audio_midi_transformer_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    if args.batch is not None:
        if not 1 <= args.batch <= 64:
            print("--batch must be 1 .. 64", file=sys.stderr)
            return 2
        wl = dataclasses.replace(wl, batch=args.batch)
    shape, B = wl.shape, wl.batch
    n_dec = wl.decode_steps if args.decode_steps is None else args.decode_steps
    R0 = wl.prefix_len + wl.n_tokens
    assert R0 + n_dec <= wl.t_cap

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: 3 x {n} bytes read and written", file=sys.stderr, flush=True)
        del src, dst
    print(f"[bench] workload {wl.key}: {wl.name}; generating weights", file=sys.stderr, flush=True)
    weights = synth.model_weights(shape, wl.model_seed)
    prefix_np = synth.workload_prefix(wl) if wl.prefix_len else None
    tokens_np = synth.workload_tokens(wl) if wl.n_tokens else None
    pairs = None
    if args.cfg is not None:
        # each sequence becomes a conditional/unconditional pair of rows
        pairs = B
        B = 2 * B
        prefix_np = synth.cfg_pair_prefix(wl) if wl.prefix_len else None
        tokens_np = np.concatenate([tokens_np] * 2) if tokens_np is not None else None
    flags = {"": 0, "a8": binding.MT_FLAG_W4A8, "f16": binding.MT_FLAG_DENSE_F16,
             "f32": binding.MT_FLAG_DENSE_F32}[variant]
    if args.phase_trace is not None:
        os.environ["MT_TRACE"] = "1"  # read when the model is created
    dec = binding.Decoder(weights, batch=B, t_cap=wl.t_cap, flags=flags)
    path = {"auto": binding.MT_DECODE_AUTO, "kernels": binding.MT_DECODE_KERNELS,
            "persistent": binding.MT_DECODE_PERSISTENT, "batched": binding.MT_DECODE_BATCHED}[args.path]
    taken = path_taken(dec, path, B)
    persistent = taken == "persistent"
    dec.set_decode_path(path)
    dev = torch.device("cuda", 0)
    prefix = torch.from_numpy(prefix_np).to(dev) if prefix_np is not None else None
    tokens = torch.from_numpy(tokens_np).to(dev) if tokens_np is not None else None
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device=dev)
    nxt = [torch.empty((B,), dtype=torch.int64, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream()
    if pairs is not None:
        guided = torch.empty((pairs, shape.vocab), dtype=torch.float32, device=dev)
        picked = torch.empty((pairs,), dtype=torch.int64, device=dev)
        row_next = torch.empty((B,), dtype=torch.int64, device=dev)

    def call(fn, *a, out):
        # one decoder call; with CFG its logits are guided and the guided
        # argmax becomes the next token of both rows of every pair
        if pairs is None:
            fn(*a, logits, out)
        else:
            fn(*a, logits, row_next)
            binding.cfg_combine(logits, args.cfg, guided=guided, next=picked, token_pair=out, stream=stream)

    def one_pass(ev=None):
        dec.reset()
        if ev is not None:
            ev["p0"].record(stream)
        call(dec.prefill, tokens, prefix, out=nxt[0])
        if ev is not None:
            ev["p1"].record(stream)
        for k in range(n_dec):
            if ev is not None and k == STEADY_FROM:
                ev["s0"].record(stream)
            if ev is not None and "per" in ev:
                ev["per"][k][0].record(stream)
            call(dec.decode_step, nxt[k & 1], out=nxt[(k + 1) & 1])
            if ev is not None and "per" in ev:
                ev["per"][k][1].record(stream)
        if ev is not None:
            ev["s1"].record(stream)

    if args.phase_trace is not None:
        if taken != "persistent" or not R0 < args.phase_trace <= wl.t_cap:
            print("--phase-trace needs the persistent path and prefix < T <= t_cap", file=sys.stderr)
            return 2
        dec.reset()
        call(dec.prefill, tokens, prefix, out=nxt[0])
        k = 0
        while dec.position < args.phase_trace:
            call(dec.decode_step, nxt[k & 1], out=nxt[(k + 1) & 1])
            k += 1
        torch.cuda.synchronize()
        dec.check()
        print(json.dumps(phase_summary(dec.debug_trace(), args.phase_trace, wl)))
        return 0

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    dec.check()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # timed passes; events around every decode call (one launch each on the
    # persistent path) give the per-launch durations for the roofline
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [dict(p0=mk(), p1=mk(), s0=mk(), s1=mk(), per=[(mk(), mk()) for _ in range(n_dec)])
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_pass(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec.check()
    prefill_ms = float(np.median([e["p0"].elapsed_time(e["p1"]) for e in evs]))
    steady_ms = float(np.mean([e["s0"].elapsed_time(e["s1"]) for e in evs]))
    n_steady = n_dec - STEADY_FROM
    ms_tok = steady_ms / n_steady
    wbytes = WEIGHT_BYTES[args.weights]
    # with CFG the guidance reads the 2Np logit rows and writes Np guided rows
    cfg_bytes = 12.0 * pairs * shape.vocab + 24.0 * pairs if pairs is not None else 0.0
    launch_bytes = np.array([step_bytes(shape, B, R0 + k + 1, wbytes) + cfg_bytes
                             for k in range(STEADY_FROM, n_dec)])
    gbps = float(launch_bytes.sum()) / (steady_ms * 1e-3) / 1e9
    step_ms = np.concatenate([np.array([a.elapsed_time(b) for a, b in e["per"]])[STEADY_FROM:] for e in evs])
    kernel_name = {"persistent": "mt_decode_step_persistent", "batched": "mt_decode_step_batched",
                   "kernels": "decode_step_kernels"}[taken]
    # the persistent step is one launch per sequence, the batched step one
    # per group of up to 8: each launch reads all weights and its own
    # sequences' cache
    groups = ([1] * B if persistent else [min(8, B - g) for g in range(0, B, 8)] if taken == "batched" else [B])
    lps = len(groups)
    step_launch_bytes = np.array([sum(step_bytes(shape, nb, R0 + k + 1, wbytes) for nb in groups)
                                  for k in range(STEADY_FROM, n_dec)]) if lps > 1 else launch_bytes
    achieved = float(step_launch_bytes.sum() * args.steps / (step_ms.sum() * 1e-3) / 1e9)
    # the counter record holds for the workload's own configuration only
    traffic = (traffic_from_profiles(kernel_name, wl.key, variant)
               if lps == 1 and pairs is None and args.batch is None else None)
    pf_flops = prefill_flops(shape, B, R0)

    # point values at T = 505, 1024 and 2048 keys (where the pass reaches them)
    all_ms = np.concatenate([np.array([a.elapsed_time(b) for a, b in e["per"]]) for e in evs])
    t_keys = np.concatenate([np.arange(n_dec) + R0 + 1] * args.steps)
    points = {str(T): round(float(all_ms[t_keys == T].mean()), 5)
              for T in (505, 1024, 2048) if np.any(t_keys == T)}
    # past the workload's last step, near the end of the cache: one prefill
    # of t_cap - 64 synthetic rows, then 16 timed decode steps (B = 1
    # workloads whose pass stops short of that)
    near_end = None
    T_far = wl.t_cap - 64
    if pairs is None and B == 1 and R0 + n_dec < T_far:
        far = torch.from_numpy(np.random.default_rng(7).standard_normal((1, T_far, shape.d_model))
                               .astype(np.float32)).to(dev)
        dec.reset()
        call(dec.prefill, None, far, out=nxt[0])
        for k in range(4):
            call(dec.decode_step, nxt[k & 1], out=nxt[(k + 1) & 1])
        far_ev = [mk() for _ in range(17)]
        far_ev[0].record(stream)
        for k in range(16):
            call(dec.decode_step, nxt[k & 1], out=nxt[(k + 1) & 1])
            far_ev[k + 1].record(stream)
        torch.cuda.synchronize()
        dec.check()
        far_ms = [far_ev[k].elapsed_time(far_ev[k + 1]) for k in range(16)]
        near_end = {"keys": f"{T_far + 5}-{T_far + 20}", "ms_per_token": round(float(np.mean(far_ms)), 5)}
        del far
    copy_gbps = measure_copy_peak(torch)

    metric = (METRIC if wl.key == "2" and args.batch is None
              else f"decode ms/token + achieved HBM GB/s, workload {wl.key}"
              + (f" at B={args.batch}" if args.batch is not None else ""))
    if pairs is not None:
        metric = (f"decode ms/token + achieved HBM GB/s, workload {wl.key} as {pairs} CFG pair(s) "
                  f"(coefficient {args.cfg:g})")
    if args.w4a8:
        metric += " (W4A8 variant)"
    elif args.weights != "int4":
        metric += f" (dense {args.weights.upper()} weights)"
    out = {
        "metric": metric,
        "value": round(ms_tok, 5),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1000.0 / args.steps, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 x i4 -> i32 projections, f32 elsewhere" if args.w4a8 else "f32",
        "weights": {"int4": "int4 symmetric RTN, group 32, fp32 scales", "f16": "dense binary16",
                    "f32": "dense binary32"}[args.weights],
        "activations": ("int8 symmetric per row and group of 32, dynamic" if args.w4a8 else "fp32"),
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) prefix; no checkpoint)",
        "config": {"workload": f"{wl.key}: {wl.name}", "layers": shape.n_layers,
                   "d_model": shape.d_model, "heads": shape.n_heads, "d_ff": shape.d_ff,
                   "vocab": shape.vocab, "batch": B, "prefix_rows": wl.prefix_len,
                   "prompt_tokens": wl.n_tokens, "decode_steps": n_dec, "t_cap": wl.t_cap,
                   "decode_path": taken,
                   **({"cfg": args.cfg, "cfg_pairs": pairs} if pairs is not None else {})},
        # guided tokens with CFG (one per pair), else one per sequence
        "decode_tokens_per_s": round((pairs if pairs is not None else B) * 1000.0 / ms_tok, 1),
        "decode_ms_per_token": {"mean": round(float(step_ms.mean()), 5),
                                "median": round(float(np.median(step_ms)), 5),
                                "p90": round(float(np.percentile(step_ms, 90)), 5)},
        "achieved_GBps": round(gbps, 1),
        "hbm_frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4),
        "decode_ms_at_T": points,
        "decode_near_cache_end": near_end,
        "hbm_frac_of_measured_copy": round(gbps / copy_gbps, 4),
        "measured_copy_GBps": round(copy_gbps, 1),
        "prefill_ms": round(prefill_ms, 3),
        ("prefill_int8_mfma_frac" if args.w4a8 else "prefill_fp32_mfma_frac"):
            round(pf_flops / (prefill_ms * 1e-3) / 1e12 / (INT8_MFMA_PEAK_TOPS if args.w4a8 else FP32_MFMA_PEAK_TFLOPS), 4),
        **({} if args.w4a8 or args.weights != "int4" else
           {"prefill_bf16x3_mfma_frac": round(pf_flops / (prefill_ms * 1e-3) / 1e12 / BF16X3_MFMA_PEAK_TFLOPS, 4)}),
        "roofline": {"kernel": kernel_name, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(float(step_launch_bytes.mean()) / lps, 1),
                     "avg_launch_us": round(float(step_ms.mean()) * 1000.0 / lps, 2),
                     "launches_per_step": lps},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, weights, prefix_np, tokens_np, w4a8=args.w4a8,
                                           dense=None if args.weights == "int4" else args.weights,
                                           cfg=args.cfg)
    dec.close()
    print(json.dumps(out), flush=True)
    return 0


def measure_copy_peak(torch, gib: int = 4, reps: int = 5) -> float:
    """Device-to-device copy of a buffer larger than the last-level cache:
    (read + written bytes) / time, best of `reps`."""
    n = gib << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * n / (best * 1e-3) / 1e9


def path_taken(dec, path: int, B: int) -> str:
    """The decode implementation the library runs for `path` (its
    MT_DECODE_AUTO rule: B <= 2 the persistent step per sequence, 3 <= B <= 16
    the batched step where supported, else the kernels)."""
    from audio_midi_transformer_amd import binding

    def ok(p):
        try:
            dec.set_decode_path(p)
        except binding.MTError:
            return False
        return True

    if path == binding.MT_DECODE_KERNELS:
        return "kernels"
    if ok(binding.MT_DECODE_BATCHED) and (path == binding.MT_DECODE_BATCHED or
                                          (path == binding.MT_DECODE_AUTO and B >= 3)):
        return "batched"
    if ok(binding.MT_DECODE_PERSISTENT) and path in (binding.MT_DECODE_AUTO, binding.MT_DECODE_PERSISTENT):
        return "persistent"
    return "kernels"


if __name__ == "__main__":
    sys.exit(main())
