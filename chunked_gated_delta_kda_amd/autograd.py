"""Differentiable entry points over libkda.

``chunk_kda`` and ``chunk_gdn`` take keyword arguments named as in the chunk_kda
call of the cuLA page ("cuLA(CUDA Linear Attention): NVIDIA Blackwell, Hopper
GPU를 위한 선형 어텐션 고성능 CUDA 커널 라이브러리", section "cuLA 설치 및
사용법"), where the output is then differentiated with ``o.backward(do)``.  The
forward pass is kda_fwd / gdn_fwd and the backward pass kda_bwd / gdn_bwd of the
C ABI; when an input needs a gradient the forward pass is kda_fwd_save /
gdn_fwd_save, which keeps in a workspace what the backward pass would otherwise
recompute, and the backward pass kda_bwd_saved / gdn_bwd_saved reuses it.  That
forward pass is the two-stage one (its records are what the backward pass
needs), so with a gradient requested o differs from kda_fwd's single-launch o
by rounding only.
This module only checks and forwards arguments (no arithmetic of the method
runs outside the library).

The kernels fix the variant the pages describe as the fast path: q and k are
L2-normalised inside, the KDA gate is formed inside from g, A_log and dt_bias
(clamped at ``lower_bound``), KDA beta arrives as logits and goes through the
sigmoid inside, and the state is [N, H, K, V].  Flags asking for anything else
are rejected.
"""
from __future__ import annotations

from . import _binding as _b


def _torch():
    import torch

    return torch


def _require(flag, want, name, what):
    if bool(flag) != want:
        raise NotImplementedError(f"{name}={flag!r} is not supported: {what}")


class _KDA:
    fn = None

    @classmethod
    def get(cls):
        if cls.fn is None:
            torch = _torch()

            class KDAFunction(torch.autograd.Function):
                @staticmethod
                def forward(ctx, q, k, v, g, beta, A_log, dt_bias, initial_state, scale,
                            lower_bound, cu_seqlens, output_final_state):
                    ctx.workspace = None
                    if any(ctx.needs_input_grad):
                        # keep what the backward pass would recompute
                        o, final, ctx.workspace = _b.kda_fwd_save(
                            q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
                            output_final_state, cu_seqlens)
                    else:
                        o, final = _b.kda_fwd(q, k, v, g, beta, A_log, dt_bias, lower_bound,
                                              scale, initial_state, output_final_state,
                                              cu_seqlens)
                    ctx.save_for_backward(q, k, v, g, beta, A_log, dt_bias, initial_state,
                                          cu_seqlens)
                    ctx.scale, ctx.lower_bound = scale, lower_bound
                    ctx.dt_shape = dt_bias.shape
                    if final is None:
                        return o
                    return o, final

                @staticmethod
                def backward(ctx, do, dfinal=None):
                    q, k, v, g, beta, A_log, dt_bias, h0, cu = ctx.saved_tensors
                    need = ctx.needs_input_grad
                    # the workspace lives as long as the graph (a second backward
                    # pass under retain_graph reuses it)
                    args = (q, k, v, g, beta, A_log, dt_bias, do.contiguous())
                    kw = dict(lower_bound=ctx.lower_bound, scale=ctx.scale, initial_state=h0,
                              dfinal=None if dfinal is None else dfinal.contiguous(),
                              cu_seqlens=cu, need_dh0=h0 is not None and need[7])
                    if ctx.workspace is not None:
                        r = _b.kda_bwd_saved(*args, ctx.workspace, **kw)
                    else:
                        r = _b.kda_bwd(*args, **kw)
                    return (r["dq"], r["dk"], r["dv"], r["dg"], r["dbeta"], r["dA_log"],
                            r["ddt_bias"].view(ctx.dt_shape), r["dh0"], None, None, None, None)

            cls.fn = KDAFunction
        return cls.fn


class _GDN:
    fn = None

    @classmethod
    def get(cls):
        if cls.fn is None:
            torch = _torch()

            class GDNFunction(torch.autograd.Function):
                @staticmethod
                def forward(ctx, q, k, v, g, beta, initial_state, scale, cu_seqlens,
                            output_final_state):
                    ctx.workspace = None
                    if any(ctx.needs_input_grad):
                        o, final, ctx.workspace = _b.gdn_fwd_save(
                            q, k, v, g, beta, scale, initial_state, output_final_state,
                            cu_seqlens)
                    else:
                        o, final = _b.gdn_fwd(q, k, v, g, beta, scale, initial_state,
                                              output_final_state, cu_seqlens)
                    ctx.save_for_backward(q, k, v, g, beta, initial_state, cu_seqlens)
                    ctx.scale = scale
                    if final is None:
                        return o
                    return o, final

                @staticmethod
                def backward(ctx, do, dfinal=None):
                    q, k, v, g, beta, h0, cu = ctx.saved_tensors
                    need = ctx.needs_input_grad
                    args = (q, k, v, g, beta, do.contiguous())
                    kw = dict(scale=ctx.scale, initial_state=h0,
                              dfinal=None if dfinal is None else dfinal.contiguous(),
                              cu_seqlens=cu, need_dh0=h0 is not None and need[5])
                    if ctx.workspace is not None:
                        r = _b.gdn_bwd_saved(*args, ctx.workspace, **kw)
                    else:
                        r = _b.gdn_bwd(*args, **kw)
                    return (r["dq"], r["dk"], r["dv"], r["dg"], r["dbeta"], r["dh0"], None, None,
                            None)

            cls.fn = GDNFunction
        return cls.fn


def chunk_kda(q, k, v, g, beta, A_log, dt_bias, scale=None, initial_state=None,
              output_final_state=False, lower_bound=-5.0, cu_seqlens=None,
              use_qk_l2norm_in_kernel=True, use_gate_in_kernel=True,
              use_beta_sigmoid_in_kernel=True, safe_gate=True, transpose_state_layout=False):
    """Differentiable chunked KDA.  q, k, g [B,T,H,K] bf16; v [B,T,H,V] bf16; beta
    logits [B,T,H] bf16; A_log [H] fp32; dt_bias [H,K] or [H*K] fp32;
    initial_state [N,H,K,V] fp32 or None; cu_seqlens int32 [N+1] or None (B = 1).
    Returns (o, final_state); final_state is None unless ``output_final_state``.
    Gradients reach q, k, v, g, beta, A_log, dt_bias and initial_state."""
    _require(use_qk_l2norm_in_kernel, True, "use_qk_l2norm_in_kernel",
             "q and k are always L2-normalised in the kernel")
    _require(use_gate_in_kernel, True, "use_gate_in_kernel",
             "the gate is always formed in the kernel from g, A_log and dt_bias")
    _require(use_beta_sigmoid_in_kernel, True, "use_beta_sigmoid_in_kernel",
             "KDA beta is taken as logits and passed through the sigmoid in the kernel")
    _require(safe_gate, True, "safe_gate", "the gate is always clamped at lower_bound")
    _require(transpose_state_layout, False, "transpose_state_layout",
             "states are [N, H, K, V]")
    if scale is None:
        scale = q.shape[-1] ** -0.5
    out = _KDA.get().apply(q, k, v, g, beta, A_log, dt_bias, initial_state, float(scale),
                           float(lower_bound), cu_seqlens, bool(output_final_state))
    return out if output_final_state else (out, None)


def chunk_gdn(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
              cu_seqlens=None, use_qk_l2norm_in_kernel=True):
    """Differentiable chunked gated delta rule (scalar gate per head and token).
    g is the fp32 log decay [B,T,H] (<= 0); beta are probabilities [B,T,H] bf16.
    Other arguments and the result as chunk_kda; gradients reach q, k, v, g, beta
    and initial_state."""
    _require(use_qk_l2norm_in_kernel, True, "use_qk_l2norm_in_kernel",
             "q and k are always L2-normalised in the kernel")
    if scale is None:
        scale = q.shape[-1] ** -0.5
    out = _GDN.get().apply(q, k, v, g, beta, initial_state, float(scale), cu_seqlens,
                           bool(output_final_state))
    return out if output_final_state else (out, None)
