"""torch.autograd integration of the MI355X attention kernels.

``attention(q, k, v, causal, sm_scale, layout)`` returns O and records the
operation for autograd: the forward saves q, k, v, O and the logsumexp, and
the backward calls ``fa_bwd`` (through the binding) for dq, dk and dv -- the
pattern of "[CS336] Assignment 2: Systems", section "FlashAttention V2" (an
autograd Function that saves L with its inputs) and of "Understanding Triton
Tutorials Part 2", section "Fused Attention 2" (``attention = _attention.apply``).
Both passes run in the library's HIP kernels; nothing is computed in PyTorch
beyond allocating outputs.
"""
import torch

from . import backward as _fa_backward
from . import forward as _fa_forward


class FlashAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal=False, sm_scale=None, layout="bhsd"):
        o, lse = _fa_forward(q, k, v, causal=causal, sm_scale=sm_scale, layout=layout)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.sm_scale = sm_scale
        ctx.layout = layout
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        # the kernels need unit dim stride and 16-byte aligned rows; autograd
        # may hand over an expanded (stride-0) gradient
        if dout.stride(-1) != 1 or any(s % 8 for s in dout.stride()):
            dout = dout.contiguous()
        dq, dk, dv = _fa_backward(q, k, v, o, dout, lse, causal=ctx.causal,
                                  sm_scale=ctx.sm_scale, layout=ctx.layout)
        return dq, dk, dv, None, None, None


def attention(q, k, v, causal=False, sm_scale=None, layout="bhsd"):
    """O = softmax(sm_scale * Q K^T [causal]) V with gradients through fa_bwd."""
    return FlashAttention.apply(q, k, v, causal, sm_scale, layout)
