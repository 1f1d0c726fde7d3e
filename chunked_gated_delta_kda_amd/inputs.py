"""Seeded synthetic inputs for the KDA / GDN forward pass.

This module is shared by the GPU tests, the benchmark and the oracle checks.
It only draws random numbers and lays them out; it holds none of the
method's arithmetic (no gate activation, normalisation or recurrence).  The
GDN recipe draws its log-decay as a clamped -softplus of a normal sample and
its beta as a sigmoid of a normal sample: those are the input distribution of
that workload, computed with torch library calls, not the method.

Shapes and dtypes follow the KDA parameter table of the FlashKDA summary
(discuss.pytorch.kr, section "FlashKDA의 KDA 연산 구조") and the usage example
of the cuLA README (section "KDA (Kimi Delta Attention) -- Blackwell (SM10X)"):
q,k,g [B,T,H,K] bf16, v [B,T,H,V] bf16, beta [B,T,H] bf16, A_log [H] fp32,
dt_bias [H,K] fp32, states fp32 [N,H,K,V], cu_seqlens int32.

Every tensor is generated on the CPU from ``torch.Generator().manual_seed``,
drawn in fp32 and rounded to bf16 (round to nearest even) where bf16.  Draw
order: sequence lengths (varlen only), q, k, v, g, beta, A_log,
initial_state.  "N(0, s)" means standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass
class Workload:
    """One synthetic problem.  All tensors live on the CPU."""
    kind: str                      # "kda" or "gdn"
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    A_log: torch.Tensor | None = None
    dt_bias: torch.Tensor | None = None
    lower_bound: float = -5.0
    scale: float = 1.0
    initial_state: torch.Tensor | None = None
    cu_seqlens: torch.Tensor | None = None
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def K(self):
        return self.q.shape[3]

    @property
    def V(self):
        return self.v.shape[3]

    @property
    def n_seqs(self):
        return self.B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def tokens(self):
        return self.B * self.T

    def to(self, device):
        """Copy of the tensors on ``device`` (a dict keyed like the binding's kwargs)."""
        d = {}
        for name in ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "initial_state",
                     "cu_seqlens"):
            t = getattr(self, name)
            d[name] = None if t is None else t.to(device)
        return d


def _normal(gen, shape, std=1.0, mean=0.0):
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std + mean


def varlen_lengths(gen, n, lo, hi):
    """n lengths uniform in [lo, hi] (inclusive)."""
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64)


def cu_from_lengths(lengths):
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.as_tensor(lengths, dtype=torch.int64), 0)
    return cu.to(torch.int32)


def kda_workload(B, T, H, K, V, seed, *, g_std=0.1, g_mean=0.0, A_log_std=0.01,
                 dt_bias_value=0.0, lower_bound=-5.0, init_std=None, lengths=None,
                 random_lengths=None, beta_mean=0.0, beta_value=None, A_log_value=None,
                 key_cos=None, key_pool=None, q_equals_k=False, name="kda"):
    """KDA inputs: q,k,v ~N(0,1) bf16; g ~N(g_mean, g_std) bf16; beta logits
    ~N(beta_mean, 1) bf16; A_log ~N(0, A_log_std) fp32; dt_bias = dt_bias_value fp32
    [H,K]; initial_state ~N(0, init_std) fp32 [N,H,K,V] or None.

    ``lengths`` (packed varlen) forces B=1 and T=sum(lengths);
    ``random_lengths=(n, lo, hi)`` draws n lengths uniform in [lo, hi] first.

    Stress variants (drawn after everything above, so the default draws are
    unchanged): ``beta_value`` / ``A_log_value`` replace the logits / A_log by a
    constant; ``key_cos=c`` makes the keys of a head share a direction, k_t =
    sqrt(c) u_h + sqrt(1 - c) z_t with u_h, z_t ~N(0, I) (pairwise cosine about
    c); ``key_pool=P`` draws each key from P fixed vectors per head (keys repeat
    within a chunk); ``q_equals_k`` sets q = k.
    """
    gen = torch.Generator().manual_seed(seed)
    if random_lengths is not None:
        lengths = varlen_lengths(gen, *random_lengths).tolist()
    cu = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = cu_from_lengths(lengths)
        B, T = 1, sum(lengths)
    N = B if cu is None else len(lengths)
    q = _normal(gen, (B, T, H, K)).to(torch.bfloat16)
    k = _normal(gen, (B, T, H, K)).to(torch.bfloat16)
    v = _normal(gen, (B, T, H, V)).to(torch.bfloat16)
    g = _normal(gen, (B, T, H, K), g_std, g_mean).to(torch.bfloat16)
    beta = _normal(gen, (B, T, H), 1.0, beta_mean).to(torch.bfloat16)
    A_log = _normal(gen, (H,), A_log_std)
    dt_bias = torch.full((H, K), float(dt_bias_value), dtype=torch.float32)
    h0 = None if init_std is None else _normal(gen, (N, H, K, V), init_std)
    if beta_value is not None:
        beta = torch.full((B, T, H), float(beta_value)).to(torch.bfloat16)
    if A_log_value is not None:
        A_log = torch.full((H,), float(A_log_value), dtype=torch.float32)
    if key_cos is not None:
        u = _normal(gen, (1, 1, H, K))
        z = _normal(gen, (B, T, H, K))
        k = (u * float(key_cos) ** 0.5 + z * (1.0 - float(key_cos)) ** 0.5).to(torch.bfloat16)
    if key_pool is not None:
        pool = _normal(gen, (H, int(key_pool), K))
        idx = torch.randint(0, int(key_pool), (B, T, H), generator=gen)
        k = pool[torch.arange(H)[None, None, :], idx].to(torch.bfloat16)
    if q_equals_k:
        q = k.clone()
    return Workload("kda", name, q, k, v, g, beta, A_log, dt_bias, float(lower_bound),
                    K ** -0.5, h0, cu)


def gdn_workload(B, T, H, K, V, seed, *, init_std=None, lengths=None, decay_shift=0.0,
                 beta_mean=0.0, beta_value=None, g_value=None, key_cos=None, key_pool=None,
                 q_equals_k=False, name="gdn"):
    """GDN inputs: q,k,v ~N(0,1) bf16; g fp32 [B,T,H] = clamp(-softplus(N(0,1) + shift), -5, 0);
    beta = sigmoid(N(beta_mean, 1)) rounded to bf16; initial_state ~N(0, init_std) or None.

    Stress variants as for kda_workload (drawn after everything above):
    ``beta_value`` (a constant probability), ``g_value`` (a constant log
    decay), ``key_cos``, ``key_pool`` and ``q_equals_k``."""
    gen = torch.Generator().manual_seed(seed)
    cu = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = cu_from_lengths(lengths)
        B, T = 1, sum(lengths)
    N = B if cu is None else len(lengths)
    q = _normal(gen, (B, T, H, K)).to(torch.bfloat16)
    k = _normal(gen, (B, T, H, K)).to(torch.bfloat16)
    v = _normal(gen, (B, T, H, V)).to(torch.bfloat16)
    g = torch.clamp(-torch.nn.functional.softplus(_normal(gen, (B, T, H)) + decay_shift),
                    -5.0, 0.0)
    beta = torch.sigmoid(_normal(gen, (B, T, H), 1.0, beta_mean)).to(torch.bfloat16)
    h0 = None if init_std is None else _normal(gen, (N, H, K, V), init_std)
    if beta_value is not None:
        beta = torch.full((B, T, H), float(beta_value)).to(torch.bfloat16)
    if g_value is not None:
        g = torch.full((B, T, H), float(g_value), dtype=torch.float32)
    if key_cos is not None:
        u = _normal(gen, (1, 1, H, K))
        z = _normal(gen, (B, T, H, K))
        k = (u * float(key_cos) ** 0.5 + z * (1.0 - float(key_cos)) ** 0.5).to(torch.bfloat16)
    if key_pool is not None:
        pool = _normal(gen, (H, int(key_pool), K))
        idx = torch.randint(0, int(key_pool), (B, T, H), generator=gen)
        k = pool[torch.arange(H)[None, None, :], idx].to(torch.bfloat16)
    if q_equals_k:
        q = k.clone()
    return Workload("gdn", name, q, k, v, g, beta, None, None, -5.0, K ** -0.5, h0, cu)


def output_grads(w: Workload, seed, *, do_std=1.0, dfinal_std=None):
    """Seeded gradients for the backward pass: dL/do ~N(0, do_std) bf16 [B,T,H,V]
    and, when ``dfinal_std`` is given, dL/d(final state) ~N(0, dfinal_std) fp32
    [N,H,K,V] (else None)."""
    gen = torch.Generator().manual_seed(seed)
    do = _normal(gen, (w.B, w.T, w.H, w.V), do_std).to(torch.bfloat16)
    dfin = None
    if dfinal_std is not None:
        dfin = _normal(gen, (w.n_seqs, w.H, w.K, w.V), dfinal_std)
    return do, dfin


# The five workloads the benchmark and the parity suite are built around.
CONFIG_NAMES = {
    0: "kda_tiny_B1_T256_H4_K64",
    1: "kda_fixed_B2_T2048_H32_K128",
    2: "kda_varlen_16seq_256to8192_H32_K128",
    3: "gdn_B4_T8192_H16_K128",
    4: "kda_long_B1_T131072_H16_K128",
}


def config(i: int) -> Workload:
    seed = 1000 + i
    name = CONFIG_NAMES[i]
    if i == 0:
        return kda_workload(1, 256, 4, 64, 64, seed, name=name)
    if i == 1:
        return kda_workload(2, 2048, 32, 128, 128, seed, init_std=0.05, name=name)
    if i == 2:
        return kda_workload(1, 0, 32, 128, 128, seed, random_lengths=(16, 256, 8192),
                            name=name)
    if i == 3:
        return gdn_workload(4, 8192, 16, 128, 128, seed, name=name)
    if i == 4:
        return kda_workload(1, 131072, 16, 128, 128, seed, init_std=0.05, name=name)
    raise KeyError(i)
