#!/usr/bin/env python3
"""Benchmark of the chunked KDA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: KDA forward, B=2, T=2048, H=32, K=V=128, bf16 q/k/v/g/beta, fp32
initial and final states (seeded synthetic inputs, chunked_gated_delta_kda_amd.
inputs.config(1)).  One step = one full forward pass (kda_prep then
kda_recur, the two stages of kda_fwd) over one batch whose inputs are already
resident in HBM.  Several input sets are rotated so that no step finds its
inputs in the 256 MB last-level cache.  Prints one JSON line.

Roofline: per-kernel durations come from HIP events recorded on the launch
stream around each stage inside the timed region (on a sample of the steps:
an event between the two kernels would lengthen every step); the dominant kernel's
algorithmic bytes (what it must read and write, see below) over its average
duration is compared with 8 TB/s.  Traffic measured with rocprofv3 counters
is read from profiles/ when it was taken on the current kernel sources.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
METRIC = "chunk_kda fwd tokens/sec, B2 T2048 H32 K=V=128; HBM GB/s & MFMA % of peak"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
C = 32  # tokens per chunk (two 16-token blocks)


# The sources that build and launch the forward kernels: a counter summary of
# the forward pass stays valid while none of them changes.
FWD_SOURCES = ("kda_api.hip", "kda_common.h", "kda_launch.h", "kda_prep.hip", "kda_recur.hip",
               "kda_split.hip")


def source_digest(names=None) -> str:
    """Hash of the kernel sources (all of them, or only `names`), comments and
    whitespace removed: a counter summary outlives edits of the comments."""
    h = hashlib.sha256()
    for p in sorted((ROOT / "chunked_gated_delta_kda_amd" / "csrc").glob("*")):
        if names is not None and p.name not in names:
            continue
        text = re.sub(r"/\*.*?\*/", " ", p.read_text(), flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(p.name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(B, T, H, K, V, N, init=True, final=True):
    """Compulsory HBM bytes of the method and of each kernel, for T a multiple of
    the chunk.  The per-(chunk, head) record holds nKG, QG and KdT (C x K bf16
    each), Aqk and Tb (C x C bf16 each) and Gamma_C (K fp32): 29184 B at K = 128."""
    th = B * T * H
    states = N * H * K * V * 4 * ((1 if init else 0) + (1 if final else 0))
    rec_per_th = (3 * C * K * 2 + 2 * C * C * 2 + K * 4) / C
    path = th * (2 * K + 2 * K + 2 * K + 2 * V + 2 + 2 * V) + states  # q k g v beta o
    prep = th * (3 * 2 * K + 2 + rec_per_th) + H * 4 + H * K * 4
    recur = th * (rec_per_th + 2 * V + 2 * V) + states
    return dict(path=path, kda_prep=prep, kda_recur=recur)


def algorithmic_flops(B, T, H, K, V):
    """Flops of the chunked method per token-head at chunk C: state read, output and
    state update (6 K V), intra-chunk products 2 C (3 K + 2 V), inverse 12 C^2."""
    return B * T * H * (6 * K * V + 2 * C * (3 * K + 2 * V) + 12 * C * C)


def measured_traffic(kernel, workload):
    """Calibrated FETCH+WRITE bytes per launch from the committed counter summary
    (profiles/<kernel>_<workload>_counters.txt), if it was taken on the current
    kernel sources; else None."""
    p = ROOT / "profiles" / f"{kernel}_{workload}_counters.txt"
    if not p.exists():
        return None
    fields = {}
    for line in p.read_text().splitlines():
        if line and not line.startswith("#") and ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("source_digest") != source_digest(FWD_SOURCES):
        return None
    return int(fields["hbm_bytes_per_launch"])


def cpu_baseline(w, budget_s):
    """The fp64 oracle on this host's cores, on whole heads of the same workload,
    repeated until about budget_s seconds of work."""
    import oracle

    orc = oracle.default()
    cores = len(os.sched_getaffinity(0))
    heads_total, done, t_total = w.H, 0, 0.0
    head = 0
    reps = 0
    while t_total < budget_s and reps < 1024:
        # one pass over `cores` heads (or all) at a time keeps every core busy
        hs = [(head + i) % heads_total for i in range(min(cores, heads_total))]
        t0 = time.perf_counter()
        orc.kda(w.q, w.k, w.v, w.g, w.beta, w.A_log, w.dt_bias, w.lower_bound, w.scale,
                w.initial_state, True, None, heads=hs, threads=cores)
        t_total += time.perf_counter() - t0
        done += len(hs)
        head = (head + len(hs)) % heads_total
        reps += 1
    tokens = w.B * w.T * done / heads_total
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 token recurrence over {done} (sequence-batch x head) passes of "
                       f"{w.B} x {w.T} tokens ({done} of {heads_total} heads per pass-set, "
                       f"{t_total:.1f} s); tokens/s scaled by heads/{heads_total}; "
                       f"input up-cast excluded")}


def bench_decode(args, torch, kda, inputs, dev):
    """One decode step (kda_decode) per timed step for N sequences x 32 heads at
    K = V = 128, the state updated in place; its bytes are the state read and
    written once plus the token's q, k, g, v, beta and o."""
    N, H, K, V = args.decode_seqs, 32, 128, 128
    w = inputs.kda_workload(N, 1, H, K, V, seed=1100, init_std=0.05, name="decode")
    d = w.to(dev)
    q, k, v, g, beta = (d[n][:, 0].contiguous() for n in ("q", "k", "v", "g", "beta"))
    state = d["initial_state"].clone()
    out = torch.empty((N, H, V), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.kda_decode(q, k, v, g, beta, d["A_log"], d["dt_bias"], w.lower_bound, w.scale,
                       state, state, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    pairs = N * H
    nbytes = pairs * (2 * K * V * 4 + 2 * K * 2 + 2 * K + 2 * V + 2 + 2 * V) + H * 4 + H * K * 4
    achieved = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "kda decode step tokens/sec (one token per sequence), H32 K=V=128",
        "value": round(N / (elapsed / args.steps), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32 state, bf16 tokens",
        "data": "synthetic",
        "config": {"workload": f"kda_decode_N{N}_H{H}_K{K}", "N": N, "H": H, "K": K, "V": V},
        "roofline": {"bound": "hbm", "kernel": "kda_decode", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": int(nbytes),
                     "avg_launch_us": round(us, 2)},
    }), flush=True)


def bench_train(args, torch, kda, inputs, dev):
    """One training step of the recurrence: the forward pass that keeps its chunk
    states (kda_fwd_save) and the backward pass that reuses them
    (kda_bwd_saved), on the benchmark workload with rotated input sets; the
    same step with the plain forward pass and the recomputing backward pass
    (kda_fwd + kda_bwd) is timed beside it."""
    base = inputs.config(1)
    B, T, H, K, V, N = base.B, base.T, base.H, base.K, base.V, base.n_seqs
    sets = []
    for r in range(args.sets):
        w = base if r == 0 else inputs.kda_workload(B, T, H, K, V, seed=1001 + 1000 * r,
                                                    init_std=0.05)
        do, dfin = inputs.output_grads(w, seed=5000 + r, dfinal_std=0.05)
        d = w.to(dev)
        d["do"], d["dfin"] = do.to(dev), dfin.to(dev)
        sets.append(d)
    ws = torch.empty(kda.bwd_workspace_size(B, T, H, K, V), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def saved_step(i):
        d = sets[i % len(sets)]
        args_ = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"])
        kda.kda_fwd_save(*args_, base.lower_bound, base.scale, d["initial_state"], workspace=ws,
                         out=out, final_out=fin)
        kda.kda_bwd_saved(*args_, d["do"], ws, base.lower_bound, base.scale, d["initial_state"],
                          d["dfin"])

    def recompute_step(i):
        d = sets[i % len(sets)]
        args_ = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"])
        kda.kda_fwd(*args_, base.lower_bound, base.scale, d["initial_state"], workspace=ws,
                    out=out, final_out=fin)
        kda.kda_bwd(*args_, d["do"], base.lower_bound, base.scale, d["initial_state"],
                    d["dfin"], workspace=ws)

    def timed(step):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps

    t_saved = timed(saved_step)
    t_recompute = timed(recompute_step)
    print(json.dumps({
        "metric": "kda training step tokens/sec (forward + all gradients), B2 T2048 H32 K=V=128",
        "value": round(B * T / t_saved, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_saved * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": inputs.CONFIG_NAMES[1] + "_train", "B": B, "T": T, "H": H, "K": K,
                   "V": V, "chunk": C, "input_sets_rotated": len(sets),
                   "step": "kda_fwd_save + kda_bwd_saved"},
        "recompute_ms_per_step": round(t_recompute * 1e3, 5),
    }), flush=True)


def bench_bwd(args, torch, kda, inputs, dev):
    """The backward pass (kda_bwd: every gradient, from dL/do and dL/d final state)
    on the benchmark workload, input sets rotated as for the forward pass.  Its
    algorithmic bytes per token-head are the reads of q, k, g, v, beta, do and the
    writes of dq, dk, dg, dv, dbeta (12 K + 6 V + 4 bytes), plus per (sequence,
    head) the initial state and the final-state gradient read and dh0 written."""
    base = inputs.config(1)
    B, T, H, K, V, N = base.B, base.T, base.H, base.K, base.V, base.n_seqs
    sets = []
    for r in range(args.sets):
        w = base if r == 0 else inputs.kda_workload(B, T, H, K, V, seed=1001 + 1000 * r,
                                                    init_std=0.05)
        do, dfin = inputs.output_grads(w, seed=5000 + r, dfinal_std=0.05)
        d = w.to(dev)
        d["do"], d["dfin"] = do.to(dev), dfin.to(dev)
        sets.append(d)
    ws = torch.empty(kda.bwd_workspace_size(B, T, H, K, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = sets[i % len(sets)]
        kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                    d["do"], base.lower_bound, base.scale, d["initial_state"], d["dfin"],
                    workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    nbytes = B * T * H * (12 * K + 6 * V + 4) + N * H * 3 * K * V * 4 + 2 * H * (K + 1) * 4
    achieved = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "kda backward tokens/sec (all gradients), B2 T2048 H32 K=V=128",
        "value": round(B * T / (elapsed / args.steps), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": inputs.CONFIG_NAMES[1] + "_bwd", "B": B, "T": T, "H": H, "K": K,
                   "V": V, "chunk": C, "input_sets_rotated": len(sets)},
        "roofline": {"bound": "hbm", "kernel": "kda_bwd (whole call, five launches)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": int(nbytes),
                     "avg_launch_us": round(us, 2)},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="instead of the forward pass, time the single-token decode step "
                         "(kda_decode) for --decode-seqs sequences x 32 heads, K=V=128")
    ap.add_argument("--decode-seqs", type=int, default=64)
    ap.add_argument("--train", action="store_true",
                    help="instead of the forward pass, time a training step (forward pass "
                         "keeping its states + backward pass reusing them) on the same workload")
    ap.add_argument("--bwd", action="store_true",
                    help="instead of the forward pass, time the backward pass (kda_bwd) on "
                         "the same workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark, copy BYTES bytes device-to-device "
                         "--steps times (the known-size reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(every (sequence, head) is independent, so a batch shards over GPUs by "
              "sequences or heads with no communication). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, str(ROOT))
    import chunked_gated_delta_kda_amd as kda
    from chunked_gated_delta_kda_amd import inputs

    kda.load()  # fails loudly if libkda.so is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "steps": args.steps}), flush=True)
        return

    if args.decode:
        bench_decode(args, torch, kda, inputs, dev)
        return
    if args.bwd:
        bench_bwd(args, torch, kda, inputs, dev)
        return
    if args.train:
        bench_train(args, torch, kda, inputs, dev)
        return

    base = inputs.config(1)
    B, T, H, K, V, N = base.B, base.T, base.H, base.K, base.V, base.n_seqs
    sets = [base.to(dev)]
    for r in range(1, args.sets):
        w = inputs.kda_workload(B, T, H, K, V, seed=1001 + 1000 * r, init_std=0.05)
        sets.append(w.to(dev))
    ws = torch.empty(kda.workspace_size(B, T, H, K, V), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # Per-kernel durations are sampled inside the timed region through the
    # stages' measurement forms (kda_prep_timed, kda_recur_timed): the kernel's
    # own start and end land in the two events, so the figure excludes the
    # dispatch gap that events recorded between kernels would add.  Every
    # PERIOD-th step times kda_prep and every PERIOD-th (offset PERIOD/2)
    # times kda_recur; the other steps launch plainly.
    period = 8 if args.steps >= 16 else 2
    def bracketed(i):
        if args.steps < 2:
            return ("prep", "recur")
        return {0: ("prep",), period // 2: ("recur",)}.get(i % period, ())

    def step(i, which=(), ev=None):
        d = sets[i % len(sets)]
        kda.kda_prep(d["q"], d["k"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                     base.lower_bound, ws, V=V, events=ev["prep"] if "prep" in which else None)
        kda.kda_recur(d["v"], K, base.scale, ws, out, d["initial_state"], fin,
                      events=ev["recur"] if "recur" in which else None)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    plan = [bracketed(i) for i in range(args.steps)]
    evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for k in which} for which in plan]
    for e in evs:  # a first record creates each event's handle (outside the timed region)
        for pair in e.values():
            for x in pair:
                x.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, plan[i], evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def mean_ms(kernel):
        t = [e[kernel][0].elapsed_time(e[kernel][1]) for e in evs if kernel in e]
        return sum(t) / len(t)

    prep_ms = mean_ms("prep")
    recur_ms = mean_ms("recur")
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms_per_step * 1e-3)

    ab = algorithmic_bytes(B, T, H, K, V, N)
    flops = algorithmic_flops(B, T, H, K, V)
    kern = {"kda_prep": prep_ms, "kda_recur": recur_ms}
    dom = max(kern, key=kern.get)
    achieved = ab[dom] / (kern[dom] * 1e-3) / 1e9
    workload = inputs.CONFIG_NAMES[1]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom, workload),
                "algorithmic_bytes_per_launch": int(ab[dom]),
                "avg_launch_us": round(kern[dom] * 1e3, 2),
                "launches_timed": sum(1 for which in plan if dom.removeprefix("kda_") in which)}
    path_s = ms_per_step * 1e-3
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "B": B, "T": T, "H": H, "K": K, "V": V, "chunk": C,
                   "input_sets_rotated": len(sets), "initial_state": "fp32 N(0,0.05)",
                   "final_state": True},
        "roofline": roofline,
        "path": {"algorithmic_bytes": int(ab["path"]),
                 "algorithmic_GBps": round(ab["path"] / path_s / 1e9, 1),
                 "hbm_frac": round(ab["path"] / path_s / 1e9 / HBM_PEAK_GBPS, 4),
                 "algorithmic_TFLOPs": round(flops / path_s / 1e12, 2),
                 "mfma_frac": round(flops / path_s / 1e12 / BF16_PEAK_TFLOPS, 5)},
        "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(base, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
