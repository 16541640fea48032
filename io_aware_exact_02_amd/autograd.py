"""torch.autograd integration of the attention library.

[ZtF] "In PyTorch": the layer above the kernels is an autograd function whose
forward saves Q, K, V, O and lse and whose backward hands them, with the
incoming dO, to the recomputing backward pass.  Both directions run in
libfa.so through the binding in this package; this module only wires the
calls into autograd (no arithmetic of its own, no fallback).

    import io_aware_exact_02_amd.autograd as faa
    out = faa.attention(q, k, v, causal=True)     # q, k, v: [B, H, T, d] bf16/fp32 on the GPU
    out.sum().backward()                            # fills q.grad, k.grad, v.grad
"""
from __future__ import annotations

import torch

from . import backward as _fa_backward
from . import forward as _fa_forward

__all__ = ["FlashAttentionFunction", "attention"]


class FlashAttentionFunction(torch.autograd.Function):
    """O = softmax(scale Q K^T [causal mask]) V; lse is kept for the backward pass."""

    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = _fa_forward(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        do = do.to(q.dtype).contiguous()
        dq, dk, dv = _fa_backward(q, k, v, o, do, lse, causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, *, causal: bool = False, scale=None):
    """Differentiable exact attention over [B, H, T, d] tensors (scale defaults to 1/sqrt(d))."""
    return FlashAttentionFunction.apply(q, k, v, bool(causal), scale)
