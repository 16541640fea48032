"""torch.autograd integration of the attention library.

[ZtF] "In PyTorch": the layer above the kernels is an autograd function whose
forward saves Q, K, V, O and lse and whose backward hands them, with the
incoming dO, to the recomputing backward pass.  Both directions run in
libfa.so through the binding in this package; this module only wires the
calls into autograd (no arithmetic of its own, no fallback).

    import io_aware_exact_02_amd.autograd as faa
    out = faa.attention(q, k, v, causal=True)     # q, k, v: [B, H, T, d] bf16/fp32 on the GPU
    out.sum().backward()                            # fills q.grad, k.grad, v.grad

A `block_mask` (uint8 [1 or H, ceil(Tq/128), ceil(Tk/128)] on the GPU) restricts
attention to the kept 128 x 128 blocks, and a `window` (wl, wr) to the keys
r - wl <= l <= r + wr of each query r, and `cu_seqlens` (int32 [ndocs + 1] on the
GPU) to the documents of packed sequences ([ZtF] "Dropout, block-sparsity, and
other real-kernel details"); both passes then run the block-sparse, window or
document kernels.
"""
from __future__ import annotations

import torch

from . import backward as _fa_backward
from . import backward_docs as _fa_backward_docs
from . import backward_masked as _fa_backward_masked
from . import backward_window as _fa_backward_window
from . import forward as _fa_forward
from . import forward_docs as _fa_forward_docs
from . import forward_masked as _fa_forward_masked
from . import forward_window as _fa_forward_window

__all__ = ["FlashAttentionFunction", "attention"]


class FlashAttentionFunction(torch.autograd.Function):
    """O = softmax(scale Q K^T [causal mask]) V; lse is kept for the backward pass."""

    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale, block_mask=None, window=None, cu_seqlens=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        ctx.docs = cu_seqlens is not None
        if cu_seqlens is not None:
            if block_mask is not None or window is not None:
                raise ValueError("cu_seqlens does not combine with a block mask or a window")
            o, lse = _fa_forward_docs(q, k, v, cu_seqlens, causal=causal, scale=scale)
            ctx.save_for_backward(q, k, v, o, lse, cu_seqlens)
        elif window is not None:
            if block_mask is not None or causal:
                raise ValueError("a window replaces causal and block masks: pass window=(-1, 0) for causal")
            o, lse = _fa_forward_window(q, k, v, window, scale=scale)
            ctx.save_for_backward(q, k, v, o, lse)
        elif block_mask is None:
            o, lse = _fa_forward(q, k, v, causal=causal, scale=scale)
            ctx.save_for_backward(q, k, v, o, lse)
        else:
            o, lse = _fa_forward_masked(q, k, v, block_mask, causal=causal, scale=scale)
            ctx.save_for_backward(q, k, v, o, lse, block_mask)
        ctx.causal, ctx.scale, ctx.masked, ctx.window = causal, scale, block_mask is not None, window
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors[:5]
        do = do.to(q.dtype).contiguous()
        if ctx.docs:
            dq, dk, dv = _fa_backward_docs(q, k, v, o, do, lse, ctx.saved_tensors[5], causal=ctx.causal,
                                           scale=ctx.scale)
        elif ctx.window is not None:
            dq, dk, dv = _fa_backward_window(q, k, v, o, do, lse, ctx.window, scale=ctx.scale)
        elif ctx.masked:
            dq, dk, dv = _fa_backward_masked(q, k, v, o, do, lse, ctx.saved_tensors[5], causal=ctx.causal,
                                             scale=ctx.scale)
        else:
            dq, dk, dv = _fa_backward(q, k, v, o, do, lse, causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, *, causal: bool = False, scale=None, block_mask=None, window=None, cu_seqlens=None):
    """Differentiable exact attention over [B, H, T, d] tensors (scale defaults to 1/sqrt(d)),
    optionally restricted to the kept blocks of `block_mask`, to a sliding `window` or to
    the documents `cu_seqlens` of packed sequences (causal within each when causal=True)."""
    return FlashAttentionFunction.apply(q, k, v, bool(causal), scale, block_mask,
                                        None if window is None else tuple(int(x) for x in window), cu_seqlens)
