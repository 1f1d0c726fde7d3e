"""Helpers shared by the GPU parity tests: run a seeded workload through the
HIP library (C ABI via the binding) and through the fp64 oracle, and compare
them with the acceptance bounds of this path.

Acceptance (for o and for final_state separately):
  ||gpu - ref||_F / ||ref||_F <= 1e-2   and   max |gpu - ref| <= 5e-2.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import chunked_gated_delta_kda_amd as kda
import oracle

REL_TOL = 1e-2
ABS_TOL = 5e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_run(w, device="cuda:0", output_final_state=True, path="fused", **kw):
    """One forward pass of w on the GPU: path "fused" is the single-launch pass
    (kda_fwd / gdn_fwd), "staged" the two-stage one (kda_fwd_split / gdn_fwd_split)."""
    d = w.to(device)
    staged = path == "staged"
    if path not in ("fused", "staged"):
        raise ValueError(path)
    if w.kind == "kda":
        fn = kda.kda_fwd_split if staged else kda.kda_fwd
        o, S = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                  w.lower_bound, w.scale, d["initial_state"], output_final_state,
                  d["cu_seqlens"], **kw)
    else:
        fn = kda.gdn_fwd_split if staged else kda.gdn_fwd
        o, S = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, d["initial_state"],
                  output_final_state, d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, S


def oracle_run(w, heads=None, threads=0):
    orc = oracle.default()
    if w.kind == "kda":
        return orc.kda(w.q, w.k, w.v, w.g, w.beta, w.A_log, w.dt_bias, w.lower_bound, w.scale,
                       w.initial_state, True, w.cu_seqlens, heads=heads, threads=threads)
    return orc.gdn(w.q, w.k, w.v, w.g, w.beta, w.scale, w.initial_state, True, w.cu_seqlens,
                   heads=heads, threads=threads)


def to64(t, heads=None, axis=None):
    if heads is not None:
        t = t.index_select(axis, torch.as_tensor(heads, device=t.device))
    return t.detach().to("cpu", torch.float64).numpy()


def errors(got, want):
    diff = got - want
    n = np.linalg.norm(want)
    rel = np.linalg.norm(diff) / n if n > 0 else np.linalg.norm(diff)
    return float(rel), float(np.max(np.abs(diff))) if diff.size else 0.0


def assert_close(name, got, want, rel_tol=REL_TOL, abs_tol=ABS_TOL):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in the GPU result"
    rel, mx = errors(got, want)
    say(f"  {name}: rel {rel:.3e} max {mx:.3e}")
    assert rel <= rel_tol, f"{name}: relative Frobenius error {rel:.3e} > {rel_tol}"
    assert mx <= abs_tol, f"{name}: max abs error {mx:.3e} > {abs_tol}"


def check_parity(w, heads=None, first_tokens=None, **kw):
    """GPU vs oracle on the same seeded inputs; ``heads`` restricts the oracle (and
    the comparison) to a subset of heads.  ``first_tokens`` adds a max-abs check on
    the first tokens of every sequence (where the initial state still matters)."""
    say(f"[parity] {w.name}: B={w.B} T={w.T} H={w.H} K={w.K} V={w.V} N={w.n_seqs}"
        f" heads={'all' if heads is None else heads} {kw if kw else ''}")
    o, S = gpu_run(w, **kw)
    ro, rS = oracle_run(w, heads)
    go = to64(o, heads, 2)
    assert_close("o", go, ro)
    if S is not None:
        assert_close("final_state", to64(S, heads, 1), rS)
    if first_tokens:
        starts = ([0] if w.cu_seqlens is None else w.cu_seqlens[:-1].tolist())
        ends = ([w.T] if w.cu_seqlens is None else w.cu_seqlens[1:].tolist())
        for a, e in zip(starts, ends):
            sl = slice(a, min(e, a + first_tokens))
            if sl.stop > sl.start:
                _, mx = errors(go[:, sl], ro[:, sl])
                assert mx <= ABS_TOL, f"max abs error {mx:.3e} in the first tokens at {a}"
    return o, S
