"""Pins for the fp64 backward oracle (``oracle/backward.py``): checks against
facts that do not come from it -- central finite differences of the pinned
C forward oracle, reverse-mode autograd through an independent PyTorch fp64
forward written here, and closed forms.

Each ``pin_*`` takes a module with the ``kda_bwd`` / ``gdn_bwd`` interface and
raises ``AssertionError`` when the pin fails.  ``tests/test_oracle_bwd.py``
runs them on the real oracle and on copies with planted mistakes, each of
which must fail at least one pin.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BIG = 1e4
EPS = 1e-6


def rel_err(got, want):
    d = np.linalg.norm(np.asarray(got) - np.asarray(want))
    n = np.linalg.norm(np.asarray(want))
    return d / n if n > 0 else d


def check(name, got, want, rtol):
    got = np.asarray(got)
    assert got.shape == np.asarray(want).shape, f"{name}: shape {got.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r = rel_err(got, want)
    assert r <= rtol, f"{name}: relative error {r:.3e} > {rtol:.1e}"


def _problem(rng, gdn, B, T, H, K, V, lengths=None, clamp=False):
    """Small fp64 inputs.  With clamp, a quarter of the gate entries sit well
    below the floor (and the rest well above), so finite differences never
    cross it."""
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    p = {
        "q": rng.standard_normal((B, T, H, K)),
        "k": rng.standard_normal((B, T, H, K)),
        "v": rng.standard_normal((B, T, H, V)),
        "cu": None if lengths is None else np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64),
    }
    N = B if lengths is None else len(lengths)
    p["h0"] = rng.standard_normal((N, H, K, V)) * 0.5
    p["do"] = rng.standard_normal((B, T, H, V))
    p["dfin"] = rng.standard_normal((N, H, K, V))
    p["scale"] = 0.6
    if gdn:
        p["g"] = -rng.uniform(0.02, 0.6, (B, T, H))
        p["beta"] = rng.uniform(0.1, 0.9, (B, T, H))
    else:
        g = rng.normal(-1.0, 1.0, (B, T, H, K))
        if clamp:
            sel = rng.random(g.shape) < 0.25
            g = np.where(sel, 6.0 + rng.random(g.shape), g)
        p["g"] = g
        p["beta"] = rng.standard_normal((B, T, H))
        p["A_log"] = rng.normal(0.0, 0.3, H)
        p["dt_bias"] = rng.normal(0.0, 0.3, (H, K))
        p["lb"] = -2.0 if clamp else -5.0
    return p


def _fwd_loss(gdn, p, over=None):
    """L = sum(o * do) + sum(S_T * dfin) from the C forward oracle."""
    x = dict(p)
    if over:
        x.update(over)
    orc = oracle.default()
    if gdn:
        o, S = orc.gdn(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["h0"], True,
                       x["cu"], threads=1)
    else:
        o, S = orc.kda(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                       x["lb"], x["scale"], x["h0"], True, x["cu"], threads=1)
    return float(np.sum(o * x["do"]) + np.sum(S * x["dfin"]))


def _fd(gdn, p, name, h=1e-6):
    base = p[name]
    grad = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        xp = base.copy()
        xm = base.copy()
        xp[idx] += h
        xm[idx] -= h
        grad[idx] = (_fwd_loss(gdn, p, {name: xp}) - _fwd_loss(gdn, p, {name: xm})) / (2 * h)
    return grad


def _bwd(mod, gdn, p, dfinal=True):
    if gdn:
        return mod.gdn_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["scale"], p["h0"],
                           p["do"], p["dfin"] if dfinal else None, p["cu"])
    return mod.kda_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], p["A_log"], p["dt_bias"],
                       p["lb"], p["scale"], p["h0"], p["do"], p["dfin"] if dfinal else None,
                       p["cu"])


KDA_NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "A_log": "dA_log",
             "dt_bias": "ddt_bias", "h0": "dh0"}
GDN_NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}


def _fd_all(mod, gdn, p, tol=1e-6):
    got = _bwd(mod, gdn, p)
    for name, gname in (GDN_NAMES if gdn else KDA_NAMES).items():
        check(f"fd {gname}", got[gname], _fd(gdn, p, name), tol)


# ---------------------------------------------------------------- finite differences
def pin_fd_kda(mod):
    """Every KDA gradient against central differences of the C forward oracle
    (two sequences, 7 tokens, initial state and a final-state gradient)."""
    _fd_all(mod, False, _problem(np.random.default_rng(101), False, 2, 7, 2, 4, 3))


def pin_fd_kda_clamp(mod):
    """The gate floor: clamped entries get zero gate gradient."""
    _fd_all(mod, False, _problem(np.random.default_rng(102), False, 1, 9, 2, 4, 3, clamp=True))


def pin_fd_gdn(mod):
    _fd_all(mod, True, _problem(np.random.default_rng(103), True, 2, 6, 2, 4, 3))


def pin_fd_varlen(mod):
    """Packed sequences (one of them empty): states reset at every boundary."""
    _fd_all(mod, False, _problem(np.random.default_rng(104), False, 1, 0, 2, 3, 2,
                                 lengths=[4, 0, 6, 1]))


# ---------------------------------------------------------------- autograd
def _torch_forward(gdn, t, p):
    """Plain PyTorch fp64 forward, written from the definition (not from the
    oracle), on tensors that require grad."""
    q, k, v = t["q"], t["k"], t["v"]
    qh = q / torch.sqrt((q * q).sum(-1, keepdim=True) + EPS)
    kh = k / torch.sqrt((k * k).sum(-1, keepdim=True) + EPS)
    if gdn:
        la = t["g"][..., None].expand(q.shape)
        b = t["beta"]
    else:
        pre = -torch.exp(t["A_log"])[None, None, :, None] * torch.nn.functional.softplus(
            t["g"] + t["dt_bias"][None, None])
        la = torch.clamp(pre, min=p["lb"])
        b = torch.sigmoid(t["beta"])
    B, T, H, K = q.shape
    outs = []
    fins = []
    for n in range(B):
        S = t["h0"][n]
        row = []
        for s in range(T):
            S = torch.exp(la[n, s])[..., None] * S
            pred = torch.einsum("hkv,hk->hv", S, kh[n, s])
            S = S + torch.einsum("hk,hv->hkv", kh[n, s], b[n, s][:, None] * (v[n, s] - pred))
            row.append(p["scale"] * torch.einsum("hkv,hk->hv", S, qh[n, s]))
        outs.append(torch.stack(row))
        fins.append(S)
    return torch.stack(outs), torch.stack(fins)


def _autograd_all(mod, gdn, p, tol):
    names = GDN_NAMES if gdn else KDA_NAMES
    t = {n: torch.tensor(p[n], dtype=torch.float64, requires_grad=True) for n in names}
    o, S = _torch_forward(gdn, t, p)
    loss = (o * torch.tensor(p["do"])).sum() + (S * torch.tensor(p["dfin"])).sum()
    loss.backward()
    got = _bwd(mod, gdn, p)
    for n, gname in names.items():
        check(f"autograd {gname}", got[gname], t[n].grad.numpy(), tol)


def pin_autograd_kda(mod):
    """Against PyTorch autograd through its own fp64 forward (40 tokens, so the
    oracle's checkpointing every 16 tokens is crossed twice)."""
    _autograd_all(mod, False, _problem(np.random.default_rng(105), False, 2, 40, 3, 8, 5,
                                       clamp=True), 1e-10)


def pin_autograd_gdn(mod):
    _autograd_all(mod, True, _problem(np.random.default_rng(106), True, 1, 33, 2, 8, 6), 1e-10)


# ---------------------------------------------------------------- closed forms
def pin_gdn_no_update_closed_form(mod):
    """beta = 0 (GDN): S_t = Gamma_t S_0, o_t = scale Gamma_t S_0^T q^_t with
    Gamma_t = exp(sum_{s<=t} g_s).  For L = sum o . do + S_T . dfin:
    dS_0 = scale sum_t Gamma_t q^_t do_t^T + Gamma_T dfin,
    dg_s = sum_{t>=s} scale Gamma_t q^_t^T S_0 do_t + [Gamma_T sum(S_0 * dfin)],
    dv = 0, dk = 0."""
    rng = np.random.default_rng(107)
    p = _problem(rng, True, 1, 8, 2, 4, 3)
    p["beta"] = np.zeros_like(p["beta"])
    got = _bwd(mod, True, p)
    qh = p["q"] / np.sqrt((p["q"] ** 2).sum(-1, keepdims=True) + EPS)
    Gam = np.exp(np.cumsum(p["g"], axis=1))  # [1,T,H]
    S0 = p["h0"][0]
    T = p["q"].shape[1]
    dS0 = np.zeros_like(S0)
    dg = np.zeros_like(p["g"])
    for h in range(S0.shape[0]):
        term = np.array([p["scale"] * Gam[0, t, h] * qh[0, t, h] @ S0[h] @ p["do"][0, t, h]
                         for t in range(T)])
        last = Gam[0, T - 1, h] * np.sum(S0[h] * p["dfin"][0, h])
        dg[0, :, h] = np.cumsum(term[::-1])[::-1] + last
        dS0[h] = sum(p["scale"] * Gam[0, t, h] * np.outer(qh[0, t, h], p["do"][0, t, h])
                     for t in range(T)) + Gam[0, T - 1, h] * p["dfin"][0, h]
    check("closed dh0", got["dh0"][0], dS0, 1e-12)
    check("closed dg", got["dg"], dg, 1e-12)
    assert np.abs(got["dv"]).max() == 0.0 and np.abs(got["dk"]).max() == 0.0


def pin_orthonormal_keys_dv(mod):
    """Decay 1, beta 1, orthonormal keys and S_0 = 0: every token writes its own
    key's slot, so S_t = sum_{s<=t} k^_s v_s^T and o_t = scale sum_{s<=t}
    (q^_t . k^_s) v_s: dv_s = scale sum_{t>=s} (q^_t . k^_s) do_t exactly
    (linear attention)."""
    rng = np.random.default_rng(108)
    T, H, K, V = 6, 2, 8, 3
    basis = np.linalg.qr(rng.standard_normal((K, K)))[0]
    k = np.stack([np.stack([basis[:, (t * 3 + h) % K] for h in range(H)]) for t in range(T)])[None]
    k = k * 1e4  # the norm epsilon is negligible
    p = _problem(rng, False, 1, T, H, K, V)
    p.update(k=k, g=np.zeros((1, T, H, K)), beta=np.full((1, T, H), BIG),
             A_log=np.full(H, -BIG), h0=np.zeros((1, H, K, V)))
    got = _bwd(mod, False, p, dfinal=False)
    qh = p["q"] / np.sqrt((p["q"] ** 2).sum(-1, keepdims=True) + EPS)
    kh = k / np.sqrt((k ** 2).sum(-1, keepdims=True) + EPS)
    want = np.zeros((1, T, H, V))
    for s in range(T):
        for t in range(s, T):
            want[0, s] += p["scale"] * np.sum(qh[0, t] * kh[0, s], -1)[:, None] * p["do"][0, t]
    check("orthonormal dv", got["dv"], want, 1e-9)


def pin_no_gradient_in_gives_zero(mod):
    """do = 0 and no final-state gradient: every gradient is exactly zero."""
    p = _problem(np.random.default_rng(109), False, 1, 5, 2, 4, 3)
    p["do"] = np.zeros_like(p["do"])
    got = _bwd(mod, False, p, dfinal=False)
    for n, g in got.items():
        assert np.all(np.asarray(g) == 0.0), n


# cheapest first (the mutation test stops at the first failing pin)
ALL_PINS = [pin_no_gradient_in_gives_zero, pin_gdn_no_update_closed_form,
            pin_orthonormal_keys_dv, pin_autograd_gdn, pin_autograd_kda, pin_fd_kda,
            pin_fd_kda_clamp, pin_fd_gdn, pin_fd_varlen]
