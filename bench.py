#!/usr/bin/env python3
"""Benchmark of the chunked KDA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1|2|3|4]

Default workload: KDA forward, B=2, T=2048, H=32, K=V=128, bf16
q/k/v/g/beta, fp32 initial and final states (seeded synthetic inputs,
chunked_gated_delta_kda_amd.inputs.config(1)).  One step = one full forward
pass over one batch whose inputs are already resident in HBM.  Several input
sets are rotated so that no step finds its inputs in the 256 MB last-level
cache.  The default 500 untimed warm-up steps give the GPU's clock time to
ramp up before the timed steps.  Prints one JSON line.

Roofline: the method's compulsory bytes (inputs read once, outputs and states
written once: 6K + 4V + 2 bytes per token-head for KDA, plus the states) over
the measured time, against 8 TB/s -- for the whole step (``path``) and for the
dominant kernel on its share of those bytes (``roofline``).  Kernel durations
come from HIP events that the kernel launch itself records, on the launch
stream, inside the timed steps.  The bytes each kernel moves by its own design
(``traffic_design``) and the HBM traffic measured with rocprofv3 counters
(``traffic``, read from profiles/ only when it was taken on the current kernel
sources) are reported beside it.
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
FWD_SOURCES = ("kda_api.hip", "kda_common.h", "kda_launch.h", "kda_ops.h", "kda_prep.hip",
               "kda_recur.hip", "kda_split.hip", "kda_fused.hip")


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
        if p.suffix == ".hip":  # and the flags it is compiled with
            from chunked_gated_delta_kda_amd.build import source_flags
            h.update(" ".join(source_flags(p.name)).encode())
    return h.hexdigest()[:16]


def method_bytes(w):
    """Compulsory HBM bytes of the method on workload ``w`` (inputs read once,
    outputs written once, no intermediates), split by what each stage of the
    two-stage path touches: the token-parallel stage reads q, k, g, beta (and
    the per-head gate parameters), the recurrence reads v and the states and
    writes o and the final states.  KDA: 6K + 4V + 2 bytes per token-head; GDN
    (fp32 log decay, bf16 beta): 4K + 4V + 6."""
    th = w.B * w.T * w.H
    K, V, H, N = w.K, w.V, w.H, w.n_seqs
    states = N * H * K * V * 4 * ((1 if w.initial_state is not None else 0) + 1)
    if w.kind == "kda":
        front = th * (3 * 2 * K + 2) + H * 4 + H * K * 4
    else:
        front = th * (2 * 2 * K + 4 + 2)
    back = th * (2 * V + 2 * V) + states
    return dict(path=front + back, kda_prep=front, kda_recur=back)


def design_bytes(w):
    """Bytes each kernel of the two-stage path moves by its own design: the
    method's bytes plus the per-(chunk, head) record that kda_prep writes and
    kda_recur reads (nKG, QG, KdT: C x K bf16 each; Aqk, Tb: C x C bf16 each;
    Gamma_C: K fp32 -- 29184 B at K = 128)."""
    K = w.K
    mb = method_bytes(w)
    n_chunks = w.H * (w.B * ((w.T + C - 1) // C) if w.cu_seqlens is None else
                      sum((int(e - b) + C - 1) // C
                          for b, e in zip(w.cu_seqlens[:-1], w.cu_seqlens[1:])))
    rec = n_chunks * (3 * C * K * 2 + 2 * C * C * 2 + K * 4)
    return dict(kda_prep=mb["kda_prep"] + rec, kda_recur=mb["kda_recur"] + rec)


def fused_design_bytes(w, seg_chunks, warm=1):
    """Bytes the single-launch kernel moves by its own design: the method's
    bytes plus the warm-up re-reads (q, k, g, beta, v of `warm` chunks before
    every segment that starts inside its sequence; one when the first
    attempt's bound holds).  Fixed-length batches only
    (seg_chunks: the segment length the launch uses)."""
    mb = method_bytes(w)
    nc = (w.T + C - 1) // C
    segs = max(1, -(-nc // seg_chunks))
    per_tok = (3 * 2 * w.K + 2 + 2 * w.V) if w.kind == "kda" else (2 * 2 * w.K + 6 + 2 * w.V)
    return mb["path"] + w.B * w.H * (segs - 1) * warm * C * per_tok


def fused_segment_chunks(w, cus=256, min_chunks=8):
    """The automatic segment length of kda_fwd for a fixed-length batch (the
    library plans for the 256 compute units of an MI355X)."""
    nc = (w.T + C - 1) // C
    pairs = w.B * w.H
    if pairs >= cus:
        return max(nc, 1)
    segs = -(-cus // pairs)
    return max(min_chunks, -(-nc // segs))


def algorithmic_flops(w):
    """Flops of the chunked method per token-head at chunk C: state read, output and
    state update (6 K V), intra-chunk products 2 C (3 K + 2 V), inverse 12 C^2."""
    K, V = w.K, w.V
    return w.B * w.T * w.H * (6 * K * V + 2 * C * (3 * K + 2 * V) + 12 * C * C)


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s):
    """The fp64 oracle on this host's cores, on whole heads of the same workload
    (every head is an independent recurrence over all the workload's
    sequences), repeated until about budget_s seconds of work; tokens/s are
    scaled from the heads done to all heads."""
    import oracle

    orc = oracle.default()
    cores = len(os.sched_getaffinity(0))
    heads_total, done, t_total = w.H, 0, 0.0
    head = 0
    reps = 0
    while t_total < budget_s and reps < 1024:
        # a batch of heads per call keeps every core busy (work items are
        # (sequence, head) pairs)
        per = max(1, min(heads_total, -(-cores // max(1, w.n_seqs))))
        hs = [(head + i) % heads_total for i in range(per)]
        t0 = time.perf_counter()
        if w.kind == "kda":
            orc.kda(w.q, w.k, w.v, w.g, w.beta, w.A_log, w.dt_bias, w.lower_bound, w.scale,
                    w.initial_state, True, w.cu_seqlens, heads=hs, threads=cores)
        else:
            orc.gdn(w.q, w.k, w.v, w.g, w.beta, w.scale, w.initial_state, True, w.cu_seqlens,
                    heads=hs, threads=cores)
        t_total += time.perf_counter() - t0
        done += len(hs)
        head = (head + len(hs)) % heads_total
        reps += 1
    tokens = w.B * w.T * done / heads_total
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": (f"fp64 token recurrence (C oracle, OpenMP over sequence x head) on "
                       f"{done} head passes over all {w.n_seqs} sequences ({w.B * w.T} tokens), "
                       f"{t_total:.1f} s; tokens/s = tokens x heads done / {heads_total} / "
                       f"seconds; input up-cast excluded")}


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


def make_sets(inputs, cfg, n_sets):
    """The workload's seeded inputs, plus n_sets - 1 more drawn the same way with
    other seeds (rotated across steps so that no step finds its inputs in the
    256 MB MALL)."""
    base = inputs.config(cfg)
    sets = [base]
    for r in range(1, n_sets):
        seed = 1000 + cfg + 1000 * r
        if cfg == 1:
            w = inputs.kda_workload(base.B, base.T, base.H, base.K, base.V, seed, init_std=0.05)
        elif cfg == 2:
            lengths = (base.cu_seqlens[1:] - base.cu_seqlens[:-1]).tolist()
            w = inputs.kda_workload(1, 0, base.H, base.K, base.V, seed, lengths=lengths)
        elif cfg == 3:
            w = inputs.gdn_workload(base.B, base.T, base.H, base.K, base.V, seed)
        else:
            w = inputs.kda_workload(base.B, base.T, base.H, base.K, base.V, seed, init_std=0.05)
        sets.append(w)
    return base, sets


def bench_fwd(args, torch, kda, inputs, dev):
    """The forward pass on one workload.  A step is one whole forward call on one
    input set: the single-launch pass kda_fwd / gdn_fwd (--path fused, the
    default) or, for the fixed-length KDA workloads, the two stages kda_prep
    then kda_recur (--path staged).  Step times come from a second pass of K
    steps with events recorded between steps (median and mean reported);
    `value` is tokens / (wall time of the K timed steps / K), timed without
    those events."""
    cfg = args.workload
    n_sets = args.sets if cfg in (1, 3) else min(args.sets, 2)
    base, host_sets = make_sets(inputs, cfg, n_sets)
    sets = [w.to(dev) for w in host_sets]
    B, T, H, K, V, N = base.B, base.T, base.H, base.K, base.V, base.n_seqs
    staged = args.path == "staged"
    if staged and (base.kind != "kda" or base.cu_seqlens is not None):
        raise SystemExit("--path staged times the fixed-length KDA workloads (1, 4)")
    if staged:
        ws_bytes = kda.workspace_size(B, T, H, K, V, N, kind=base.kind, segment_chunks=-1,
                                      path="staged")
    else:
        ws_bytes = kda.workspace_size(B, T, H, K, V, N, kind=base.kind)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # Per-kernel durations: every PERIOD-th step launches its kernel(s) through
    # the measurement forms (kda_fwd_timed / gdn_fwd_timed for the single
    # launch, kda_prep_timed and (offset PERIOD/2) kda_recur_timed for the
    # stages): the kernel's own start and end land in the two events, so no
    # dispatch gap is counted.
    period = 8 if args.steps >= 16 else 2
    names = ("prep", "recur") if staged else ("fused",)

    def bracketed(i):
        if args.steps < 2:
            return names
        if staged:
            return {0: ("prep",), period // 2: ("recur",)}.get(i % period, ())
        return ("fused",) if i % (period // 2) == 0 else ()

    def step(i, which=(), ev=None):
        d = sets[i % len(sets)]
        if staged:
            kda.kda_prep(d["q"], d["k"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                         base.lower_bound, ws, V=V, events=ev["prep"] if "prep" in which else None)
            kda.kda_recur(d["v"], K, base.scale, ws, out, d["initial_state"], fin,
                          events=ev["recur"] if "recur" in which else None)
            return
        e = ev["fused"] if "fused" in which else None
        if base.kind == "kda":
            kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                        base.lower_bound, base.scale, d["initial_state"], True, d["cu_seqlens"],
                        workspace=ws, out=out, final_out=fin, events=e)
        else:
            kda.gdn_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], base.scale,
                        d["initial_state"], True, d["cu_seqlens"], workspace=ws, out=out,
                        final_out=fin, events=e)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    plan = [bracketed(i) for i in range(args.steps)]
    evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for k in which} for which in plan]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e in evs:  # a first record creates each event's handle (outside the timed region)
        for pair in e.values():
            for x in pair:
                x.record(stream)
    # timed region: K plain steps between two synchronisations (the value)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the same K steps again with an event between consecutive steps (step
    # times: median) and the sampled per-kernel events
    for i in range(args.steps):
        marks[i].record(stream)
        step(args.warmup + i, plan[i], evs[i])
    marks[-1].record(stream)
    torch.cuda.synchronize()

    step_us = sorted(marks[i].elapsed_time(marks[i + 1]) * 1e3 for i in range(args.steps))
    median_us = step_us[len(step_us) // 2] if len(step_us) % 2 else \
        0.5 * (step_us[len(step_us) // 2 - 1] + step_us[len(step_us) // 2])
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms_per_step * 1e-3)

    mb = method_bytes(base)
    flops = algorithmic_flops(base)
    workload = inputs.CONFIG_NAMES[cfg]
    line = {
        "metric": METRIC if cfg == 1 else
        f"{base.kind}_fwd tokens/sec, {workload}; HBM GB/s & MFMA % of peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "B": B, "T": T, "H": H, "K": K, "V": V, "N": N,
                   "chunk": C, "path": args.path, "input_sets_rotated": len(sets),
                   "initial_state": None if base.initial_state is None else "fp32 N(0,0.05)",
                   "final_state": True},
        "step_us": {"median": round(median_us, 2), "mean": round(sum(step_us) / len(step_us), 2),
                    "min": round(step_us[0], 2), "max": round(step_us[-1], 2)},
    }
    # the method's bytes over the median step: the whole path against 8 TB/s
    path_s = median_us * 1e-6
    line["path"] = {"method_bytes": int(mb["path"]),
                    "method_GBps": round(mb["path"] / path_s / 1e9, 1),
                    "hbm_frac": round(mb["path"] / path_s / 1e9 / HBM_PEAK_GBPS, 4),
                    "algorithmic_TFLOPs": round(flops / path_s / 1e12, 2),
                    "mfma_frac": round(flops / path_s / 1e12 / BF16_PEAK_TFLOPS, 5)}

    def mean_ms(kernel):
        t = [e[kernel][0].elapsed_time(e[kernel][1]) for e in evs if kernel in e]
        return sum(t) / len(t)

    if staged:
        db = design_bytes(base)
        kern = {"kda_prep": mean_ms("prep"), "kda_recur": mean_ms("recur")}
        dom = max(kern, key=kern.get)
        algo, design = mb[dom], db[dom]
    else:
        kern = {"kda_fused": mean_ms("fused")}
        dom = "kda_fused"
        algo = mb["path"]
        design = (fused_design_bytes(base, fused_segment_chunks(base))
                  if base.cu_seqlens is None else None)
    achieved = algo / (kern[dom] * 1e-3) / 1e9
    line["roofline"] = {
        "bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": measured_traffic(dom, workload),
        "algorithmic_bytes_per_launch": int(algo),
        "traffic_design": None if design is None else int(design),
        "avg_launch_us": round(kern[dom] * 1e3, 2),
        "launches_timed": sum(1 for which in plan if dom.removeprefix("kda_") in which)}
    line["kernels_us"] = {k: round(v * 1e3, 2) for k, v in kern.items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(base, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first: about 30 ms of work at the default workload, "
                         "so that the GPU's clock has ramped up (5 steps measured 15%% slower)")
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
    ap.add_argument("--workload", type=int, default=1, choices=(1, 2, 3, 4),
                    help="forward workload (configuration index of inputs.config): 1 is the "
                         "benchmark line; 2 (packed KDA), 3 (GDN), 4 (long KDA) time the same "
                         "call on the other parity workloads")
    ap.add_argument("--path", choices=("fused", "staged"), default="fused",
                    help="forward path: the single launch kda_fwd (default) or the two "
                         "stages kda_prep + kda_recur (fixed-length KDA workloads)")
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

    bench_fwd(args, torch, kda, inputs, dev)


if __name__ == "__main__":
    main()
