"""chunk_kda / chunk_gdn under torch autograd: the gradients that o.backward()
produces are those of kda_bwd / gdn_bwd called directly (bit for bit: the same
kernels on the same inputs, and the kernels are deterministic), and they match
the fp64 backward oracle."""
import pytest
import torch

import chunked_gated_delta_kda_amd as kda
from chunked_gated_delta_kda_amd import inputs
from chunked_gated_delta_kda_amd.autograd import chunk_gdn, chunk_kda
from oracle import backward as obwd
from test_gpu_bwd import close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def leaf(t, dtype=None):
    return t.to(DEV, dtype=dtype or t.dtype).detach().requires_grad_(True)


def kda_case():
    w = inputs.kda_workload(1, 100, 2, 64, 64, seed=31, dt_bias_value=-6.0, init_std=0.05)
    do, dfin = inputs.output_grads(w, seed=32, dfinal_std=0.05)
    return w, do, dfin


@pytest.mark.parametrize("final", [True, False])
def test_chunk_kda_backward_is_kda_bwd(final):
    w, do, dfin = kda_case()
    args = dict(q=leaf(w.q), k=leaf(w.k), v=leaf(w.v), g=leaf(w.g), beta=leaf(w.beta),
                A_log=leaf(w.A_log), dt_bias=leaf(w.dt_bias.reshape(-1)),
                initial_state=leaf(w.initial_state))
    o, S = chunk_kda(**args, scale=w.scale, output_final_state=final, lower_bound=w.lower_bound)
    assert (S is not None) == final
    outs, grads = [o], [do.to(DEV)]
    if final:
        outs.append(S)
        grads.append(dfin.to(DEV))
    torch.autograd.backward(outs, grads)
    d = w.to(DEV)
    ref = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                      do.to(DEV), w.lower_bound, w.scale, d["initial_state"],
                      dfin.to(DEV) if final else None)
    torch.cuda.synchronize()
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                      ("A_log", "dA_log"), ("initial_state", "dh0")):
        assert torch.equal(args[name].grad, ref[key]), name
    assert torch.equal(args["dt_bias"].grad, ref["ddt_bias"].reshape(-1))


def test_chunk_kda_gradients_match_oracle():
    w, do, dfin = kda_case()
    args = dict(q=leaf(w.q), k=leaf(w.k), v=leaf(w.v), g=leaf(w.g), beta=leaf(w.beta),
                A_log=leaf(w.A_log), dt_bias=leaf(w.dt_bias), initial_state=leaf(w.initial_state))
    o, S = chunk_kda(**args, scale=w.scale, output_final_state=True, lower_bound=w.lower_bound)
    torch.autograd.backward([o, S], [do.to(DEV), dfin.to(DEV)])
    ref = obwd.kda_bwd(w.q, w.k, w.v, w.g, w.beta, w.A_log, w.dt_bias, w.lower_bound, w.scale,
                       w.initial_state, do, dfin)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                      ("initial_state", "dh0")):
        close(key, args[name].grad.double().cpu().numpy(), ref[key])


def test_chunk_gdn_backward_is_gdn_bwd():
    w = inputs.gdn_workload(1, 90, 2, 64, 64, seed=33, init_std=0.05)
    do, dfin = inputs.output_grads(w, seed=34, dfinal_std=0.05)
    args = dict(q=leaf(w.q), k=leaf(w.k), v=leaf(w.v), g=leaf(w.g), beta=leaf(w.beta),
                initial_state=leaf(w.initial_state))
    o, S = chunk_gdn(**args, scale=w.scale, output_final_state=True)
    torch.autograd.backward([o, S], [do.to(DEV), dfin.to(DEV)])
    d = w.to(DEV)
    ref = kda.gdn_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do.to(DEV), w.scale,
                      d["initial_state"], dfin.to(DEV))
    torch.cuda.synchronize()
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                      ("initial_state", "dh0")):
        assert torch.equal(args[name].grad, ref[key]), name


def test_chunk_kda_backward_twice_with_retained_graph():
    w, do, dfin = kda_case()
    q = leaf(w.q)
    rest = dict(k=leaf(w.k), v=leaf(w.v), g=leaf(w.g), beta=leaf(w.beta), A_log=leaf(w.A_log),
                dt_bias=leaf(w.dt_bias), initial_state=leaf(w.initial_state))
    o, _ = chunk_kda(q=q, **rest, scale=w.scale, lower_bound=w.lower_bound)
    o.backward(do.to(DEV), retain_graph=True)
    g1 = q.grad.clone()
    q.grad = None
    o.backward(do.to(DEV))
    assert torch.equal(q.grad, g1)
