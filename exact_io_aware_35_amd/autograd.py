"""torch.autograd glue over the C ABI: the forward saves O and the LSE, and the
backward recomputes P from the LSE through fa_backward (no N x N tensor is ever
kept). Argument marshalling only, like binding.py."""

from __future__ import annotations

import torch

from . import binding


class FlashAttention(torch.autograd.Function):
    """out = attention(q, k, v) with the gradients of fa_backward.

    q, k, v: [batch, seqlen, heads, headdim] bf16 device tensors (the backward
    is built for bf16). Only out carries a gradient; the LSE is returned for
    inspection and is marked non-differentiable.
    """

    @staticmethod
    def forward(ctx, q, k, v, causal=False, window=(-1, -1), softmax_scale=None, seqlens_k=None,
                alibi_slopes=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, lse = binding.forward(q, k, v, causal=causal, window=window,
                                   softmax_scale=softmax_scale, seqlens_k=seqlens_k,
                                   alibi_slopes=alibi_slopes)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.opts = dict(causal=causal, window=window, softmax_scale=softmax_scale,
                        seqlens_k=seqlens_k, alibi_slopes=alibi_slopes)
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv = binding.backward(q, k, v, out, lse, dout.contiguous(), **ctx.opts)
        return dq, dk, dv, None, None, None, None, None


def flash_attention(q, k, v, causal=False, window=(-1, -1), softmax_scale=None, seqlens_k=None,
                    alibi_slopes=None):
    """Differentiable attention output [batch, seqlen, heads, headdim] (the LSE is dropped)."""
    out, _ = FlashAttention.apply(q, k, v, causal, tuple(window), softmax_scale, seqlens_k,
                                  alibi_slopes)
    return out
