"""GPU parity of the decode step (kda_decode / gdn_decode, through the C ABI)
against the fp64 oracle: one step equals the token recurrence over one
token, and T steps in a row (state updated in place) equal the recurrence
over those T tokens."""
import numpy as np
import pytest
import torch

import chunked_gated_delta_kda_amd as kda
from chunked_gated_delta_kda_amd import inputs
from parity_util import assert_close, gpu_run, oracle_run, say, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _step_inputs(d, w, t):
    """Token t of every sequence as [N, H, *] device tensors."""
    q = d["q"][:, t].contiguous()
    k = d["k"][:, t].contiguous()
    v = d["v"][:, t].contiguous()
    beta = d["beta"][:, t].contiguous()
    g = d["g"][:, t].contiguous()
    return q, k, v, g, beta


def _decode(d, w, t, state, state_out=None):
    q, k, v, g, beta = _step_inputs(d, w, t)
    if w.kind == "kda":
        return kda.kda_decode(q, k, v, g, beta, d["A_log"], d["dt_bias"], w.lower_bound,
                              w.scale, state, state_out)
    return kda.gdn_decode(q, k, v, g, beta, w.scale, state, state_out)


def _workload(kind, N, T, H, K, V, seed):
    if kind == "kda":
        return inputs.kda_workload(N, T, H, K, V, seed=seed, dt_bias_value=-6.0, init_std=0.05)
    return inputs.gdn_workload(N, T, H, K, V, seed=seed, init_std=0.05, decay_shift=-6.0)


@pytest.mark.parametrize("kind", ["kda", "gdn"])
@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_decode_one_step(kind, K, V):
    w = _workload(kind, 3, 1, 5, K, V, seed=5000 + K + V + (kind == "gdn"))
    say(f"[decode] {kind} one step N=3 H=5 K={K} V={V}")
    d = w.to(DEV)
    o, S = _decode(d, w, 0, d["initial_state"])
    torch.cuda.synchronize()
    ro, rS = oracle_run(w)
    assert_close("o", to64(o), ro[:, 0])
    assert_close("state", to64(S), rS)


@pytest.mark.parametrize("kind", ["kda", "gdn"])
def test_decode_steps_in_place_equal_recurrence(kind):
    """40 steps, the state updated in place, equal the recurrence over 40 tokens
    (and the chunked forward pass over them)."""
    T = 40
    w = _workload(kind, 2, T, 4, 128, 128, seed=5100 + (kind == "gdn"))
    say(f"[decode] {kind} {T} steps in place")
    d = w.to(DEV)
    state = d["initial_state"].clone()
    outs = []
    for t in range(T):
        o, _ = _decode(d, w, t, state, state_out=state)
        outs.append(o)
    torch.cuda.synchronize()
    o_all = torch.stack(outs, 1)  # [N, T, H, V]
    ro, rS = oracle_run(w)
    assert_close("o", to64(o_all), ro)
    assert_close("state", to64(state), rS)
    fo, fS = gpu_run(w)
    assert_close("o vs forward", to64(o_all), to64(fo))
    assert_close("state vs forward", to64(state), to64(fS))


def test_decode_after_prefill():
    """kda_fwd over T tokens, then one decode step from its final state, equals
    the recurrence over T + 1 tokens."""
    T = 97
    w = _workload("kda", 2, T + 1, 3, 128, 128, seed=5200)
    pre = inputs.Workload("kda", "prefill", w.q[:, :T].contiguous(), w.k[:, :T].contiguous(),
                          w.v[:, :T].contiguous(), w.g[:, :T].contiguous(),
                          w.beta[:, :T].contiguous(), w.A_log, w.dt_bias, w.lower_bound,
                          w.scale, w.initial_state)
    _, S = gpu_run(pre)
    d = w.to(DEV)
    o, S2 = _decode(d, w, T, S)
    torch.cuda.synchronize()
    ro, rS = oracle_run(w)
    assert_close("o", to64(o), ro[:, T])
    assert_close("state", to64(S2), rS)


def test_decode_zero_state_equals_none():
    w = _workload("kda", 2, 1, 3, 128, 64, seed=5300)
    d = w.to(DEV)
    o1, S1 = _decode(d, w, 0, None)
    o2, S2 = _decode(d, w, 0, torch.zeros_like(d["initial_state"]))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_decode_clamp_active():
    # the gate floor binds on nearly every channel
    w = inputs.kda_workload(2, 1, 4, 128, 128, seed=5400, g_mean=8.0, g_std=1.0, init_std=0.05)
    d = w.to(DEV)
    o, S = _decode(d, w, 0, d["initial_state"])
    torch.cuda.synchronize()
    ro, rS = oracle_run(w)
    assert_close("o", to64(o), ro[:, 0])
    assert_close("state", to64(S), rS)


def test_decode_many_pairs():
    """Many (sequence, head) pairs in one launch, as in batched serving."""
    w = _workload("kda", 64, 1, 32, 128, 128, seed=5500)
    d = w.to(DEV)
    o, S = _decode(d, w, 0, d["initial_state"])
    torch.cuda.synchronize()
    heads = [0, 17, 31]
    ro, rS = oracle_run(w, heads=heads)
    assert_close("o", to64(o, heads, 1), ro[:, 0])
    assert_close("state", to64(S, heads, 1), rS)
