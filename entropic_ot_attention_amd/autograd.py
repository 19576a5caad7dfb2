"""torch.autograd wrapper of the library's forward and tail VJP (argument marshalling only).

SinkhornAttention.apply(Q, K, V, W, T, R, epsilon, schedule) runs sinkhorn_attn_fwd on
[bh, L, d] device tensors and keeps the saved duals and output; its backward runs
sinkhorn_attn_vjp with the incoming cotangent (and that output), so a model built with torch ops trains through the HIP kernels
[technical summaries §2.1-§2.2: stopped base, differentiable tail, exact tail VJP].
"""

from __future__ import annotations

import torch

from . import binding as B


class SinkhornAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, W: int, T: int, R: int = 2, epsilon: float = 1.0,
                schedule: str = "one_reference"):
        O, duals = B.forward(Q, K, V, W, T, R, epsilon)
        ctx.save_for_backward(Q, K, V, duals, O)
        ctx.cfg = (W, T, R, epsilon, schedule)
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, duals, O = ctx.saved_tensors
        W, T, R, epsilon, schedule = ctx.cfg
        dQ, dK, dV = B.vjp(Q, K, V, duals, dO.contiguous().to(Q.dtype), W, T, R, epsilon,
                           schedule=schedule, O=O)
        return dQ, dK, dV, None, None, None, None, None


def sinkhorn_attention(Q, K, V, W: int, T: int, R: int = 2, epsilon: float = 1.0,
                       schedule: str = "one_reference"):
    return SinkhornAttention.apply(Q, K, V, W, T, R, epsilon, schedule)
