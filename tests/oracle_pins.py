"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself -- closed forms, invariants, a textbook filter routine, brute
force, an independent chunkwise algorithm and hand-worked examples.

Each ``pin_*`` takes an object with the ``oracle.Oracle`` interface
(``kda(...)`` and ``gdn(...)``) and raises ``AssertionError`` when the pin
fails.  ``tests/test_oracle_pins.py`` runs them on the real oracle and
``tests/test_oracle_mutants.py`` runs them on copies of the oracle with
planted mistakes, each of which must fail at least one pin.

The pages print no equations and no values (see ``oracle/kda_oracle.c`` for
the reading).  Inputs are chosen so the quantities a pin needs are known by
construction: softplus(log(expm1(m))) = m exactly in real arithmetic, so
g = log(expm1(m)) with A_log = 0 and dt_bias = 0 gives decay exp(-m);
A_log = -1e4 gives a zero decay rate (decay 1); beta logits of +-1e4 give
beta 1 and 0; logit(p) gives beta p.  Where the pin's closed form needs unit
keys, the keys are scaled to norm >= 1000 so that the normalisation epsilon
(1e-6) moves results by < 1e-12 relative; one pin measures that epsilon.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.signal import lfilter

from oracle.chunked import chunked_forward

BIG = 1e4
LN2 = float(np.log(2.0))
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def logit(p):
    p = np.asarray(p, dtype=np.float64)
    return np.log(p) - np.log1p(-p)


def pre_activation_for(m):
    """g with softplus(g) = m (m > 0)."""
    return np.log(np.expm1(np.asarray(m, dtype=np.float64)))


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rel_err(got, want):
    d = np.linalg.norm(np.asarray(got) - np.asarray(want))
    n = np.linalg.norm(np.asarray(want))
    return d / n if n > 0 else d


def check(name, got, want, rtol):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r = rel_err(got, want)
    assert r <= rtol, f"{name}: relative error {r:.3e} > {rtol:.1e}"


def big_rows(rng, shape, lo=1e3, hi=1e4):
    """Random directions with norms in [lo, hi] along the last axis."""
    x = unit(rng.standard_normal(shape))
    return x * rng.uniform(lo, hi, shape[:-1] + (1,))


def no_decay(H):
    return np.full(H, -BIG)


# --------------------------------------------------------------------------- gate
def pin_decay_per_head(orc):
    """beta = 0: S_t = Diag(Gamma_t) S_0 and o_t = scale * S_0^T (Gamma_t * q^_t).
    With g = dt_bias = 0, softplus(0) = ln 2 and A_log[h] sets the rate exp(A_log[h]),
    so the decay is 2^-rate: 1/2, 1/4 and 1/sqrt(2) for A_log = 0, ln 2, -ln 2."""
    rng = np.random.default_rng(11)
    B, T, H, K, V = 1, 6, 3, 4, 3
    q = np.zeros((B, T, H, K))
    for t in range(T):
        q[0, t, :, t % K] = 1000.0
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = np.zeros((B, T, H, K))
    beta = np.full((B, T, H), -BIG)
    A_log = np.array([0.0, LN2, -LN2])
    S0 = rng.standard_normal((1, H, K, V))
    o, S = orc.kda(q, k, v, g, beta, A_log, np.zeros((H, K)), -5.0, 0.7, S0)
    alpha = np.array([0.5, 0.25, 2 ** -0.5])
    want = np.zeros_like(o)
    for t in range(T):
        for h in range(H):
            want[0, t, h] = 0.7 * alpha[h] ** (t + 1) * S0[0, h, t % K]
    check("decay_per_head o", o, want, 1e-11)
    check("decay_per_head final", S, alpha[None, :, None, None] ** T * S0, 1e-12)


def pin_decay_per_channel_bias(orc):
    """dt_bias[h,c] = log(expm1(m[h,c])) with g = 0 gives log decay -rate_h * m[h,c]
    per channel; beta = 0 so o_t = scale * sum_c q^_tc exp(-(t+1) rate_h m_hc) S_0[c,:]."""
    rng = np.random.default_rng(12)
    B, T, H, K, V = 2, 5, 2, 5, 3
    m = 0.1 * (np.arange(K)[None, :] + 1) + 0.3 * np.arange(H)[:, None]
    dt = pre_activation_for(m)
    A_log = np.array([0.0, np.log(3.0)])
    rate = np.array([1.0, 3.0])
    q = big_rows(rng, (B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    S0 = rng.standard_normal((B, H, K, V))
    o, S = orc.kda(q, k, v, np.zeros((B, T, H, K)), np.full((B, T, H), -BIG), A_log, dt,
                   -5.0, 1.3, S0)
    qn = unit(q)
    want = np.zeros_like(o)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                gam = np.exp(-(t + 1) * rate[h] * m[h])
                want[b, t, h] = 1.3 * (qn[b, t, h] * gam) @ S0[b, h]
    check("decay_per_channel o", o, want, 1e-10)
    wantS = np.exp(-T * rate[None, :, None] * m[None])[..., None] * S0
    check("decay_per_channel final", S, wantS, 1e-12)


def pin_decay_from_gate_with_clamp(orc):
    """Time-varying per-channel gate g = log(expm1(m)); entries with g = 40 have
    softplus ~ 40 and hit the floor: log decay = max(lb, -rate * m)."""
    rng = np.random.default_rng(13)
    B, T, H, K, V = 1, 7, 2, 4, 3
    m = rng.uniform(0.05, 1.5, (B, T, H, K))
    clamp = rng.random((B, T, H, K)) < 0.25
    g = np.where(clamp, 40.0, pre_activation_for(m))
    m_eff = np.where(clamp, 40.0, m)
    lb = -2.0
    A_log = np.array([0.0, LN2])
    rate = np.array([1.0, 2.0])
    log_a = np.maximum(lb, -rate[None, None, :, None] * m_eff)
    Gam = np.exp(np.cumsum(log_a, axis=1))
    q = big_rows(rng, (B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    S0 = rng.standard_normal((1, H, K, V))
    o, S = orc.kda(q, k, v, g, np.full((B, T, H), -BIG), A_log, np.zeros((H, K)), lb, 1.0, S0)
    want = np.einsum("bthk,bhkv->bthv", unit(q) * Gam, S0)
    check("gate_clamp o", o, want, 1e-10)
    check("gate_clamp final", S, Gam[:, -1][..., None] * S0, 1e-12)


# --------------------------------------------------------------------------- beta, norm
def pin_beta_sigmoid(orc):
    """One token, no decay, zero state: S_1 = beta k^ v^T and, with q = k,
    o_1 = scale * beta * v.  Logits 0, ln 3, -ln 3, logit(.9), logit(.01)."""
    rng = np.random.default_rng(14)
    p = np.array([0.5, 0.75, 0.25, 0.9, 0.01])
    B, T, H, K, V = len(p), 1, 1, 6, 4
    k = big_rows(rng, (B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    beta = logit(p).reshape(B, T, H)
    o, S = orc.kda(k, k, v, np.zeros((B, T, H, K)), beta, no_decay(H), np.zeros((H, K)),
                   -5.0, 0.9)
    check("beta o", o, 0.9 * p[:, None, None, None] * v, 1e-11)
    wantS = p[:, None, None, None] * np.einsum("bk,bv->bkv", unit(k[:, 0, 0]), v[:, 0, 0])[:, None]
    check("beta final", S, wantS, 1e-11)


def pin_norm_epsilon(orc):
    """|k|^2 = 1e-6 equals the epsilon under the square root, so k^ = k / sqrt(2e-6)
    has squared norm 1/2, and with q = k, beta = 1, no decay, zero state:
    o_1 = scale * (q^ . k^) v = scale * v / 2."""
    B, T, H, K, V = 1, 1, 1, 3, 2
    k = np.zeros((B, T, H, K))
    k[..., 1] = 1e-3
    v = np.array([3.0, -2.0]).reshape(B, T, H, V)
    o, S = orc.kda(k, k, v, np.zeros((B, T, H, K)), np.full((B, T, H), BIG), no_decay(H),
                   np.zeros((H, K)), -5.0, 1.0)
    check("eps o", o, 0.5 * v, 1e-9)
    wantS = np.zeros((1, 1, K, V))
    wantS[0, 0, 1] = v[0, 0, 0] / np.sqrt(2.0)
    check("eps final", S, wantS, 1e-9)


# --------------------------------------------------------------------------- delta rule
def pin_retrieval(orc):
    """Delta-rule retrieval: with beta = 1 the update makes S_t^T k^_t = v_t whatever
    the decay and the previous state, so with q = k, o_t = scale * v_t."""
    rng = np.random.default_rng(15)
    B, T, H, K, V = 2, 9, 2, 5, 4
    k = big_rows(rng, (B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    S0 = rng.standard_normal((B, H, K, V))
    beta = np.full((B, T, H), BIG)
    for A_log, g in ((no_decay(H), np.zeros((B, T, H, K))),
                     (rng.normal(0, 0.3, H), rng.normal(0, 1, (B, T, H, K)))):
        o, _ = orc.kda(k, k, v, g, beta, A_log, np.zeros((H, K)), -5.0, 0.5, S0)
        check("retrieval o", o, 0.5 * v, 1e-9)


def pin_orthogonal_keys_linear_attention(orc):
    """No decay and mutually orthogonal keys k_t = c_t e_{pi(t)}: the delta correction
    only removes what S_0 stores for that key, so
    o = scale * (Q^ S_0 + tril(Q^ K^T) diag(beta) (V - K^ S_0)) -- causal linear attention."""
    rng = np.random.default_rng(16)
    B, T, H, K, V = 1, 6, 1, 6, 4
    perm = rng.permutation(K)
    k = np.zeros((B, T, H, K))
    for t in range(T):
        k[0, t, 0, perm[t]] = rng.uniform(100, 1000) * rng.choice([-1, 1])
    q = big_rows(rng, (B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    p = rng.uniform(0.05, 0.95, (B, T, H))
    S0 = rng.standard_normal((B, H, K, V))
    o, S = orc.kda(q, k, v, np.zeros((B, T, H, K)), logit(p), no_decay(H), np.zeros((H, K)),
                   -5.0, 0.8, S0)
    Q, Kn, Vm, b = unit(q[0, :, 0]), unit(k[0, :, 0]), v[0, :, 0], p[0, :, 0]
    R = Vm - Kn @ S0[0, 0]
    want = 0.8 * (Q @ S0[0, 0] + np.tril(Q @ Kn.T) @ (b[:, None] * R))
    check("orthogonal o", o[0, :, 0], want, 1e-10)
    check("orthogonal final", S[0, 0], S0[0, 0] + Kn.T @ (b[:, None] * R), 1e-10)


def pin_small_beta_limit(orc):
    """No decay, beta = eps: to first order in eps,
    o = scale * (Q^ S_0 + eps * tril(Q^ K^T) (V - K^ S_0))."""
    rng = np.random.default_rng(17)
    B, T, H, K, V = 1, 12, 1, 5, 3
    eps = 1e-7
    q, k = big_rows(rng, (B, T, H, K)), big_rows(rng, (B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    S0 = rng.standard_normal((B, H, K, V))
    o, _ = orc.kda(q, k, v, np.zeros((B, T, H, K)), np.full((B, T, H), logit(eps)),
                   no_decay(H), np.zeros((H, K)), -5.0, 1.0, S0)
    Q, Kn, Vm = unit(q[0, :, 0]), unit(k[0, :, 0]), v[0, :, 0]
    base = Q @ S0[0, 0]
    first = np.tril(Q @ Kn.T) @ (Vm - Kn @ S0[0, 0])
    check("small beta first order", (o[0, :, 0] - base) / eps, first, 1e-5)


def pin_scalar_state_filter(orc):
    """K = 1: the state is a scalar per value column and the recurrence is the
    first-order linear filter s_t = a s_{t-1} + beta k^_t v_t with
    a = alpha (1 - beta k^_t^2); scipy.signal.lfilter computes it."""
    rng = np.random.default_rng(18)
    B, T, H, K, V = 1, 40, 1, 1, 3
    sk = rng.choice([-1.0, 1.0], (B, T, H, K))
    sq = rng.choice([-1.0, 1.0], (B, T, H, K))
    k, q = 1000.0 * sk, 1000.0 * sq
    v = rng.standard_normal((B, T, H, V))
    pbeta, m = 0.3, 0.2
    S0 = rng.standard_normal((1, 1, 1, V))
    o, S = orc.kda(q, k, v, np.full((B, T, H, K), pre_activation_for(m)),
                   np.full((B, T, H), logit(pbeta)), np.zeros(H), np.zeros((H, K)), -5.0,
                   1.0, S0)
    kn2 = 1e6 / (1e6 + 1e-6)
    a = np.exp(-m) * (1.0 - pbeta * kn2)
    khat = sk[0, :, 0, 0] * np.sqrt(kn2)
    want = np.zeros((T, V))
    last = np.zeros(V)
    for j in range(V):
        x = pbeta * khat * v[0, :, 0, j]
        y, zf = lfilter([1.0], [1.0, -a], x, zi=[a * S0[0, 0, 0, j]])
        want[:, j] = y
        last[j] = y[-1]
    qhat = sq[0, :, 0, 0] * np.sqrt(kn2)
    check("scalar filter o", o[0, :, 0], qhat[:, None] * want, 1e-11)
    check("scalar filter final", S[0, 0, 0], last, 1e-11)


def pin_brute_force_products(orc):
    """Tiny case by explicit K x K matrices: S_t = M_t S_{t-1} + beta_t k^_t v_t^T with
    M_t = (I - beta_t k^_t k^_t^T) Diag(alpha_t), alpha and beta known by construction."""
    rng = np.random.default_rng(19)
    B, T, H, K, V = 2, 5, 2, 3, 2
    m = rng.uniform(0.01, 2.0, (B, T, H, K))
    p = rng.uniform(0.05, 0.95, (B, T, H))
    q, k = big_rows(rng, (B, T, H, K)), big_rows(rng, (B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    S0 = rng.standard_normal((B, H, K, V))
    o, S = orc.kda(q, k, v, pre_activation_for(m), logit(p), np.zeros(H), np.zeros((H, K)),
                   -5.0, 1.1, S0)
    for b in range(B):
        for h in range(H):
            St = S0[b, h].copy()
            for t in range(T):
                kk = unit(k[b, t, h])
                M = (np.eye(K) - p[b, t, h] * np.outer(kk, kk)) @ np.diag(np.exp(-m[b, t, h]))
                St = M @ St + p[b, t, h] * np.outer(kk, v[b, t, h])
                check("brute o", o[b, t, h], 1.1 * St.T @ unit(q[b, t, h]), 1e-11)
            check("brute final", S[b, h], St, 1e-11)


# --------------------------------------------------------------------------- chunk form
def _random_kda(rng, B, T, H, K, V, init=True, decay=-4.0):
    return dict(q=rng.standard_normal((B, T, H, K)), k=rng.standard_normal((B, T, H, K)),
                v=rng.standard_normal((B, T, H, V)),
                g=rng.normal(0, 1.0, (B, T, H, K)),
                beta=rng.standard_normal((B, T, H)),
                A_log=rng.normal(0, 0.5, H),
                dt_bias=rng.normal(decay, 1.0, (H, K)),
                initial_state=(rng.normal(0, 0.5, (B, H, K, V)) if init else None))


def pin_chunk_sizes_agree(orc):
    """The chunkwise WY algorithm (independent NumPy code) at chunk 1, 16 and 64
    equals the token recurrence, with ragged last chunks and a varlen batch."""
    rng = np.random.default_rng(20)
    B, T, H, K, V = 2, 150, 2, 8, 6
    d = _random_kda(rng, B, T, H, K, V)
    ref_o, ref_S = orc.kda(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                           d["dt_bias"], -5.0, 0.6, d["initial_state"])
    for C in (1, 16, 64):
        o, S = chunked_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                               d["dt_bias"], -5.0, 0.6, d["initial_state"], chunk=C)
        check(f"chunk{C} o", ref_o, o, 1e-9)
        check(f"chunk{C} final", ref_S, S, 1e-9)
    cu = np.array([0, 37, 37, 120, 300])
    dv = _random_kda(rng, 1, 300, H, K, V, init=False)
    h0 = rng.normal(0, 0.5, (4, H, K, V))
    ref_o, ref_S = orc.kda(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["A_log"],
                           dv["dt_bias"], -5.0, 0.6, h0, cu_seqlens=cu)
    for C in (16, 64):
        o, S = chunked_forward(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["A_log"],
                               dv["dt_bias"], -5.0, 0.6, h0, cu_seqlens=cu, chunk=C)
        check(f"varlen chunk{C} o", ref_o, o, 1e-9)
        check(f"varlen chunk{C} final", ref_S, S, 1e-9)
    # GDN through the chunk form as well
    g = -rng.uniform(0.0, 0.3, (B, T, H))
    pb = rng.uniform(0.05, 0.95, (B, T, H))
    ref_o, ref_S = orc.gdn(d["q"], d["k"], d["v"], g, pb, 0.6, d["initial_state"])
    o, S = chunked_forward(d["q"], d["k"], d["v"], g, pb, scale=0.6,
                           initial_state=d["initial_state"], chunk=16, gdn=True)
    check("gdn chunk16 o", ref_o, o, 1e-9)
    check("gdn chunk16 final", ref_S, S, 1e-9)


# --------------------------------------------------------------------------- invariants
def pin_state_continuation(orc):
    """run(0:T) equals run(T1:T) started from run(0:T1)'s final state."""
    rng = np.random.default_rng(21)
    B, T, H, K, V = 2, 50, 2, 6, 5
    d = _random_kda(rng, B, T, H, K, V)
    args = lambda sl: (d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["g"][:, sl],
                       d["beta"][:, sl], d["A_log"], d["dt_bias"], -5.0, 0.9)
    full_o, full_S = orc.kda(*args(slice(0, T)), d["initial_state"])
    for T1 in (16, 23):
        o1, S1 = orc.kda(*args(slice(0, T1)), d["initial_state"])
        o2, S2 = orc.kda(*args(slice(T1, T)), S1)
        check(f"continuation@{T1} o", np.concatenate([o1, o2], axis=1), full_o, 1e-13)
        check(f"continuation@{T1} final", S2, full_S, 1e-13)


def pin_varlen_equals_separate(orc):
    """A packed batch equals separate runs, each sequence starting from its own
    state; an empty sequence returns its initial state."""
    rng = np.random.default_rng(22)
    H, K, V = 2, 5, 4
    cu = np.array([0, 7, 7, 30, 64])
    d = _random_kda(rng, 1, 64, H, K, V, init=False)
    h0 = rng.normal(0, 0.5, (4, H, K, V))
    o, S = orc.kda(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], -5.0,
                   0.7, h0, cu_seqlens=cu)
    for n in range(4):
        a, e = cu[n], cu[n + 1]
        if e == a:
            assert np.array_equal(S[n], h0[n]), "empty sequence must keep its state"
            continue
        sl = slice(a, e)
        on, Sn = orc.kda(d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["g"][:, sl],
                         d["beta"][:, sl], d["A_log"], d["dt_bias"], -5.0, 0.7, h0[n:n + 1])
        assert np.array_equal(o[:, sl], on), f"varlen output of sequence {n}"
        assert np.array_equal(S[n:n + 1], Sn), f"varlen state of sequence {n}"


def pin_value_columns_independent(orc):
    """Columns of S evolve independently: splitting V gives the same numbers."""
    rng = np.random.default_rng(23)
    B, T, H, K, V = 1, 20, 2, 4, 6
    d = _random_kda(rng, B, T, H, K, V)
    o, S = orc.kda(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], -5.0,
                   0.7, d["initial_state"])
    for sl in (slice(0, 2), slice(2, 6)):
        o2, S2 = orc.kda(d["q"], d["k"], np.ascontiguousarray(d["v"][..., sl]), d["g"],
                         d["beta"], d["A_log"], d["dt_bias"], -5.0, 0.7,
                         np.ascontiguousarray(d["initial_state"][..., sl]))
        assert np.array_equal(o[..., sl], o2) and np.array_equal(S[..., sl], S2)


def pin_gdn_is_scalar_gate_kda(orc):
    """GDN with log decay -m_t per head equals KDA whose gate gives decay exp(-m_t) on
    every channel; GDN takes beta as a probability, KDA as a logit."""
    rng = np.random.default_rng(24)
    B, T, H, K, V = 2, 11, 2, 5, 3
    m = rng.uniform(0.01, 3.0, (B, T, H))
    p = rng.uniform(0.05, 0.95, (B, T, H))
    q, k = rng.standard_normal((B, T, H, K)), rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    S0 = rng.standard_normal((B, H, K, V))
    og, Sg = orc.gdn(q, k, v, -m, p, 0.4, S0)
    gk = np.broadcast_to(pre_activation_for(m)[..., None], (B, T, H, K))
    ok, Sk = orc.kda(q, k, v, gk, logit(p), np.zeros(H), np.zeros((H, K)), -5.0, 0.4, S0)
    check("gdn vs kda o", og, ok, 1e-12)
    check("gdn vs kda final", Sg, Sk, 1e-12)


def pin_gdn_decay_closed_form(orc):
    """GDN with beta = 0: o_t = scale * exp(sum_{s<=t} g_s) S_0^T q^_t."""
    rng = np.random.default_rng(25)
    B, T, H, K, V = 1, 8, 3, 4, 3
    g = -rng.uniform(0.0, 1.0, (B, T, H))
    q = big_rows(rng, (B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    S0 = rng.standard_normal((B, H, K, V))
    o, S = orc.gdn(q, k, v, g, np.zeros((B, T, H)), 1.5, S0)
    Gam = np.exp(np.cumsum(g, axis=1))
    want = 1.5 * Gam[..., None] * np.einsum("bthk,bhkv->bthv", unit(q), S0)
    check("gdn closed form o", o, want, 1e-11)
    check("gdn closed form final", S, Gam[:, -1][..., None, None] * S0, 1e-12)


# --------------------------------------------------------------------------- hand-worked
def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_hand_worked(orc):
    """Two-token, K = V = 2 examples worked by hand (tests/golden/hand_worked.json)."""
    cases = load_golden("hand_worked.json")["cases"]
    for c in cases:
        a = {key: (np.array(val, dtype=np.float64) if isinstance(val, list) else val)
             for key, val in c["inputs"].items()}
        if c["kind"] == "kda":
            o, S = orc.kda(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
                           a["lower_bound"], a["scale"], a.get("initial_state"))
        else:
            o, S = orc.gdn(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"],
                           a.get("initial_state"))
        check(f"{c['name']} o", o, np.array(c["expected"]["o"]), 1e-10)
        check(f"{c['name']} final", S, np.array(c["expected"]["final_state"]), 1e-10)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
