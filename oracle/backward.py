"""Reverse-mode pass (gradients) of the gated delta rule in fp64 NumPy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Nothing in the GPU
library may import or call this module.

Given the forward inputs, dL/do and optionally dL/d(final state) of some
scalar loss L, it returns dL/d(every input) of the forward pass defined in
``kda_oracle.c``:

  q^_t = q_t / n_q,  n_q = sqrt(sum_c q_tc^2 + eps)        (k^ likewise)
  KDA: x = g + dt_bias[h],  a = -exp(A_log[h]) softplus(x),
       log a_t = max(lb, a),  b_t = sigmoid(beta_logit_t)
  GDN: log a_t = g_t (every channel),  b_t = beta_t
  S_t = (I - b_t k^_t k^_t^T) Diag(a_t) S_{t-1} + b_t k^_t v_t^T,
  o_t = scale S_t^T q^_t.

The pages show the backward only as autograd over the forward call (cuLA
README mirror, section "Usage": q, k, v created with requires_grad and
o.backward(do); the roadmap lists backward kernels for training, and the
FlashQLA summary describes separate forward and backward functions for custom
training loops).  They print no gradient formula, so the oracle is the plain
definition: reverse-mode differentiation of the token recurrence, one step
at a time.  One forward step, with S the incoming state, is

  w = Diag(a) S,  r = w^T k^,  u = b (v - r),  S' = w + k^ u^T,  o = scale S'^T q^

and its adjoint, with dS the gradient reaching S' (from later tokens and
from o):

  dS  += scale q^ do^T;         dq^ = scale S' do
  dk^  = dS u + w dr;           du = dS^T k^;   dv = b du;   db = du . (v - r)
  dr   = -b du;                 dw = dS + k^ dr^T
  da   = rowsum(dw * S);        dS_prev = Diag(a) dw

followed by the chain rule through the L2 norms, the gate and the sigmoid.
Readings where the definition leaves a choice:
  - the floor max(lb, x) passes the gradient where x >= lb and blocks it
    where the floor is active (x < lb), the convention of a clamp;
  - GDN's dg is the sum over channels of d(log a) (one gate per token and
    head); GDN's beta gradient is with respect to the probability it takes.
States are kept every CHECKPOINT tokens and recomputed in between.
"""
from __future__ import annotations

import numpy as np

NORM_EPS = 1e-6
CHECKPOINT = 16


def _f64(x):
    if x is None:
        return None
    if type(x).__module__.startswith("torch"):
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _norm(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)
    return x / n, n


def _norm_grad(xh, n, dxh):
    """Gradient through x^ = x / sqrt(|x|^2 + eps)."""
    return (dxh - xh * np.sum(xh * dxh, axis=-1, keepdims=True)) / n


def _step(S, qh, kh, a, b, v, scale):
    """One forward token step for P pairs at once; returns the pieces the
    adjoint needs.  S [P,K,V], qh/kh/a [P,K], b [P], v [P,V]."""
    w = a[:, :, None] * S
    r = np.einsum("pkv,pk->pv", w, kh)
    u = b[:, None] * (v - r)
    Sn = w + kh[:, :, None] * u[:, None, :]
    return w, r, u, Sn


def core_backward(qh, kh, la, b, v, do, S0, dST, scale):
    """Adjoint of the recurrence over one sequence for P independent pairs.

    qh, kh, la: [P,T,K] (normalised q, k and log decay), b [P,T], v and do
    [P,T,V], S0 and dST [P,K,V] (dST may be None).  Returns (dqh, dkh, dla,
    db, dv, dS0) with the shapes of (qh, kh, la, b, v, S0)."""
    P, T, K = qh.shape
    V = v.shape[-1]
    a = np.exp(la)
    # forward sweep: states entering every CHECKPOINT-th token
    ck = {}
    S = S0.copy()
    for t in range(T):
        if t % CHECKPOINT == 0:
            ck[t] = S.copy()
        S = _step(S, qh[:, t], kh[:, t], a[:, t], b[:, t], v[:, t], scale)[3]
    dqh = np.zeros_like(qh)
    dkh = np.zeros_like(kh)
    dla = np.zeros_like(la)
    db = np.zeros_like(b)
    dv = np.zeros_like(v)
    dS = np.zeros((P, K, V)) if dST is None else dST.copy()
    for seg in range((T - 1) // CHECKPOINT * CHECKPOINT if T else -1, -1, -CHECKPOINT):
        end = min(seg + CHECKPOINT, T)
        prev = [ck[seg]]  # prev[i] = state entering token seg + i
        for t in range(seg, end - 1):
            prev.append(_step(prev[-1], qh[:, t], kh[:, t], a[:, t], b[:, t], v[:, t], scale)[3])
        for t in range(end - 1, seg - 1, -1):
            Sp = prev[t - seg]
            w, r, u, Sn = _step(Sp, qh[:, t], kh[:, t], a[:, t], b[:, t], v[:, t], scale)
            # o_t = scale S_t^T q^_t
            dS = dS + scale * qh[:, t, :, None] * do[:, t, None, :]
            dqh[:, t] = scale * np.einsum("pkv,pv->pk", Sn, do[:, t])
            # S_t = w + k^ u^T
            du = np.einsum("pkv,pk->pv", dS, kh[:, t])
            dk = np.einsum("pkv,pv->pk", dS, u)
            # u = b (v - r)
            dv[:, t] = b[:, t, None] * du
            db[:, t] = np.sum(du * (v[:, t] - r), axis=-1)
            dr = -b[:, t, None] * du
            # r = w^T k^
            dw = dS + kh[:, t, :, None] * dr[:, None, :]
            dk = dk + np.einsum("pkv,pv->pk", w, dr)
            dkh[:, t] = dk
            # w = Diag(a) S_{t-1}
            dla[:, t] = np.sum(dw * Sp, axis=-1) * a[:, t]
            dS = a[:, t, :, None] * dw
    return dqh, dkh, dla, db, dv, dS


def _spans(B, T, cu):
    if cu is None:
        return [(n, 0, T) for n in range(B)]
    cu = [int(x) for x in np.asarray(_f64(cu)).astype(np.int64)]
    return [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def _heads(x, heads, axis):
    return x if x is None or heads is None else np.take(x, list(heads), axis=axis)


def _run(gdn, q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state, do,
         dfinal, cu_seqlens, heads):
    q, k, v, g, beta, do = (_heads(_f64(x), heads, 2) for x in (q, k, v, g, beta, do))
    initial_state = _heads(_f64(initial_state), heads, 1)
    dfinal = _heads(_f64(dfinal), heads, 1)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    qh, nq = _norm(q)
    kh, nk = _norm(k)
    if gdn:
        la = np.broadcast_to(g[..., None], (B, T, H, K)).copy()
        b = beta
    else:
        A_log = _heads(_f64(A_log), heads, 0)
        dt = _heads(_f64(dt_bias).reshape(-1, K), heads, 0)
        x = g + dt[None, None]
        rate = np.exp(A_log)[None, None, :, None]
        a_pre = -rate * _softplus(x)
        la = np.maximum(lower_bound, a_pre)
        b = _sigmoid(beta)
    spans = _spans(B, T, cu_seqlens)
    N = len(spans)
    h0 = np.zeros((N, H, K, V)) if initial_state is None else _f64(initial_state)
    dfin = None if dfinal is None else _f64(dfinal)
    dqh = np.zeros_like(q)
    dkh = np.zeros_like(k)
    dla = np.zeros((B, T, H, K))
    db = np.zeros((B, T, H))
    dv = np.zeros_like(v)
    dh0 = np.zeros((N, H, K, V))
    for i, (row, t0, t1) in enumerate(spans):
        sl = (row, slice(t0, t1))

        def ph(x):  # [len, H, ...] -> [H, len, ...]
            return np.ascontiguousarray(np.moveaxis(x[sl], 1, 0))

        res = core_backward(ph(qh), ph(kh), ph(la), ph(b), ph(v), ph(do), h0[i].copy(),
                            None if dfin is None else dfin[i].copy(), scale)
        for dst, src in zip((dqh, dkh, dla, db, dv), res[:5]):
            dst[sl] = np.moveaxis(src, 0, 1)
        dh0[i] = res[5]
    out = {"dq": _norm_grad(qh, nq, dqh), "dk": _norm_grad(kh, nk, dkh), "dv": dv, "dh0": dh0}
    if gdn:
        out["dg"] = dla.sum(axis=-1)
        out["dbeta"] = db
    else:
        da = np.where(a_pre >= lower_bound, dla, 0.0)
        dx = da * (-rate * _sigmoid(x))
        out["dg"] = dx
        out["ddt_bias"] = dx.sum(axis=(0, 1))
        out["dA_log"] = (da * a_pre).sum(axis=(0, 1, 3))
        out["dbeta"] = db * b * (1.0 - b)
    return out


def kda_bwd(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state, do,
            dfinal=None, cu_seqlens=None, heads=None):
    """Gradients of the KDA forward pass: dict with dq, dk, dv, dg (pre-activation
    gate), dbeta (logits), dA_log [H], ddt_bias [H,K], dh0 [N,H,K,V].  ``heads``
    restricts every input and result to those head indices."""
    return _run(False, q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                do, dfinal, cu_seqlens, heads)


def gdn_bwd(q, k, v, g, beta, scale, initial_state, do, dfinal=None, cu_seqlens=None,
            heads=None):
    """Gradients of the GDN forward pass: dict with dq, dk, dv, dg [B,T,H]
    (log decay), dbeta [B,T,H] (probabilities), dh0 [N,H,K,V]."""
    return _run(True, q, k, v, g, beta, None, None, 0.0, scale, initial_state, do, dfinal,
                cu_seqlens, heads)

