"""Chunkwise (WY / UT-transform) form of the gated delta rule in fp64 NumPy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is a second, independent algorithm for the same recurrence as
``kda_oracle.c``.  The FlashKDA summary on discuss.pytorch.kr (sections
"Flash Linear Attention과 비교" and "커널 퓨전(Kernel Fusion) 전략의 분리")
describes processing tokens in chunks of 16 with a small lower-triangular
matrix inverse per chunk; FLA's default chunk is 64.  Within a chunk of n
tokens, with Gamma_r = prod_{s<=r} a_s (per channel) the running decay:

  A[r,j]   = beta_r * sum_c k^_rc Gamma_rc k^_jc / Gamma_jc      (j < r, else 0)
  T        = (I + A)^-1
  W        = T diag(beta) (K^ * Gamma)          U = T diag(beta) V
  U'       = U - W S_0                          (true per-token updates)
  Aqk[r,j] = sum_c q^_rc Gamma_rc k^_jc / Gamma_jc                  (j <= r)
  O        = scale * ((Q^ * Gamma) S_0 + Aqk U')
  S_n      = Diag(Gamma_n) S_0 + (K^ * Gamma_n / Gamma)^T U'

It follows from unrolling S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T over
the chunk; the inverse is a library solve (no blocking or doubling here).
With chunk=1 it reduces to the token recurrence step by step.
"""
from __future__ import annotations

import numpy as np

NORM_EPS = 1e-6


def l2_normalise(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)


def softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def kda_log_decay(g, A_log, dt_bias, lower_bound):
    """Per-channel log decay [B,T,H,K] from the pre-activation gate."""
    H, K = g.shape[2], g.shape[3]
    dt = np.asarray(dt_bias, dtype=np.float64).reshape(H, K)
    rate = np.exp(np.asarray(A_log, dtype=np.float64))[None, None, :, None]
    return np.maximum(lower_bound, -rate * softplus(g + dt[None, None]))


def chunked_forward(q, k, v, g, beta, A_log=None, dt_bias=None, lower_bound=-5.0,
                    scale=None, initial_state=None, cu_seqlens=None, chunk=16, gdn=False,
                    output_final_state=True, record=None):
    """Same arguments and results as ``Oracle.kda`` / ``Oracle.gdn``.

    ``record``, if a list, receives one dict per (sequence, head, chunk) with
    the chunk-level intermediates (A, T, W, U, Aqk, Gamma, U').
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    qn, kn = l2_normalise(q), l2_normalise(k)
    if gdn:
        log_a = np.broadcast_to(g[..., None], (B, T, H, K))
        b_all = beta
    else:
        log_a = kda_log_decay(g, A_log, dt_bias, lower_bound)
        b_all = sigmoid(beta)
    if cu_seqlens is None:
        spans = [(n, 0, T) for n in range(B)]
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        spans = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    N = len(spans)
    o = np.zeros((B, T, H, V))
    final = np.zeros((N, H, K, V))
    for n, (b, t0, t1) in enumerate(spans):
        for h in range(H):
            S = (np.zeros((K, V)) if initial_state is None
                 else np.array(initial_state[n, h], dtype=np.float64))
            for s in range(t0, t1, chunk):
                e = min(s + chunk, t1)
                m = e - s
                Kc, Qc, Vc = kn[b, s:e, h], qn[b, s:e, h], v[b, s:e, h]
                bc = b_all[b, s:e, h]
                G = np.cumsum(log_a[b, s:e, h], axis=0)       # [m,K] log Gamma
                Gam, Ginv = np.exp(G), np.exp(-G)
                A = np.tril((bc[:, None] * (Kc * Gam)) @ (Kc * Ginv).T, -1)
                Tm = np.linalg.solve(np.eye(m) + A, np.eye(m))
                W = Tm @ (bc[:, None] * (Kc * Gam))
                U = Tm @ (bc[:, None] * Vc)
                Up = U - W @ S
                Aqk = np.tril((Qc * Gam) @ (Kc * Ginv).T)
                o[b, s:e, h] = scale * ((Qc * Gam) @ S + Aqk @ Up)
                Kdec = Kc * np.exp(G[-1][None, :] - G)
                S_new = np.exp(G[-1])[:, None] * S + Kdec.T @ Up
                if record is not None:
                    record.append(dict(seq=n, head=h, start=s, A=A, T=Tm, W=W, U=U, Aqk=Aqk,
                                       Gamma=Gam, Uprime=Up, S_in=S.copy(), S_out=S_new))
                S = S_new
            final[n, h] = S
    return o, (final if output_final_state else None)
