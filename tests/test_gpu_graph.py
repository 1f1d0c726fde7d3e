"""The C-ABI calls allocate nothing, synchronise nothing and record no memset,
so they can be captured in a HIP graph when the caller supplies the workspace
and the outputs.  Each test captures a call, replays it several times with
eager work and synchronisation in between, and requires every replay to equal
the eager result bit for bit (the kernels are deterministic)."""
import pytest
import torch

import chunked_gated_delta_kda_amd as kda
from chunked_gated_delta_kda_amd import inputs
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def capture(fn):
    """Warm up on a side stream (as torch requires), then capture fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("varlen", [False, True])
def test_forward_graph_replays_equal_eager(varlen):
    if varlen:
        w = inputs.kda_workload(1, 0, 2, 128, 128, seed=71, dt_bias_value=-6.0, init_std=0.05,
                                lengths=[40, 1, 100, 64])
    else:
        w = inputs.kda_workload(2, 150, 2, 128, 128, seed=72, dt_bias_value=-6.0, init_std=0.05)
    d = w.to(DEV)
    cu = d.get("cu_seqlens")
    B, T, H, K = d["q"].shape
    V = d["v"].shape[-1]
    N = w.n_seqs
    ws = torch.empty(kda.workspace_size(B, T, H, K, V, N), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=DEV)
    fin = torch.empty((N, H, K, V), dtype=torch.float32, device=DEV)

    def call():
        kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                    w.lower_bound, w.scale, d["initial_state"], cu_seqlens=cu, workspace=ws,
                    out=out, final_out=fin)

    call()
    torch.cuda.synchronize()
    o_ref, s_ref = out.clone(), fin.clone()
    g = capture(call)
    for r in range(REPLAYS):
        out.fill_(float("nan"))  # eager work between replays
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}: o equal {torch.equal(out, o_ref)}, state equal {torch.equal(fin, s_ref)}")
        assert torch.equal(out, o_ref) and torch.equal(fin, s_ref)


def test_backward_graph_replays_equal_eager():
    w = inputs.kda_workload(1, 100, 2, 64, 64, seed=73, dt_bias_value=-6.0, init_std=0.05)
    do, dfin = inputs.output_grads(w, seed=74, dfinal_std=0.05)
    d = w.to(DEV)
    do, dfin = do.to(DEV), dfin.to(DEV)
    ws = torch.empty(kda.bwd_workspace_size(w.B, w.T, w.H, w.K, w.V), dtype=torch.uint8, device=DEV)
    res = {}

    def call():
        res["g"] = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                               d["dt_bias"], do, w.lower_bound, w.scale, d["initial_state"], dfin,
                               workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in res["g"].items() if v is not None}
    g = capture(call)
    outs = res["g"]  # the graph's own output buffers
    for r in range(REPLAYS):
        for v in outs.values():
            if v is not None:
                v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(outs[k], v), f"replay {r}: {k}"


def test_decode_loop_in_a_graph_equals_eager_steps():
    """A serving loop: one decode step captured once, replayed for each new
    token, state updated in place."""
    N, H, K, V, steps = 8, 4, 128, 128, 5
    w = inputs.kda_workload(N, steps, H, K, V, seed=75, init_std=0.05)
    d = w.to(DEV)
    tok = {n: torch.empty_like(d[n][:, 0]) for n in ("q", "k", "v", "g", "beta")}
    state = d["initial_state"].clone()
    out = torch.empty((N, H, V), dtype=torch.bfloat16, device=DEV)

    def step():
        kda.kda_decode(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], d["A_log"],
                       d["dt_bias"], w.lower_bound, w.scale, state, state, out)

    # eager reference
    ref_state = d["initial_state"].clone()
    ref_out = []
    for t in range(steps):
        o, ref_state = kda.kda_decode(*(d[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")),
                                      d["A_log"], d["dt_bias"], w.lower_bound, w.scale,
                                      ref_state, ref_state)
        ref_out.append(o.clone())
    torch.cuda.synchronize()
    for n in tok:
        tok[n].copy_(d[n][:, 0])
    saved = state.clone()
    g = capture(step)  # the warm-up and the capture ran once on the stream: undo the warm-up
    state.copy_(saved)
    for t in range(steps):
        for n in tok:
            tok[n].copy_(d[n][:, t])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out[t]), f"step {t}: output"
    assert torch.equal(state, ref_state)
