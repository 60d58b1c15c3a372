"""Attention as a torch.autograd.Function over the library's kernels.

Forward runs ``dash_attn_fwd`` (O and the log-sum-exp); backward runs
``dash_attn_bwd`` with the chosen schedule, so a model built from this op gets
bitwise-reproducible attention gradients with any deterministic schedule
("Resumo Técnico: DASH ...", §1 and §3: deterministic backward inside
end-to-end training).  This module only marshals tensors; every step runs in
the library.
"""
from __future__ import annotations

import torch

from .attention import AUTO, attn_bwd, attn_fwd


class DashAttentionFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale: float, schedule: int):
        o, lse = attn_fwd(q, k, v, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale, ctx.schedule = causal, scale, schedule
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, o, do.contiguous(), lse, ctx.causal, ctx.schedule, scale=ctx.scale)
        return dq, dk, dv, None, None, None


def dash_attention(q, k, v, causal: bool = False, scale: float = 0.0, schedule: int = AUTO):
    """softmax(scale Q K^T [+ causal]) V for contiguous bf16 [B, H, S, D] tensors
    (K and V may have fewer heads: grouped-query attention); scale 0 = 1/sqrt(D)."""
    return DashAttentionFunction.apply(q, k, v, causal, scale, schedule)
