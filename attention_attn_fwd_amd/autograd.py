"""Autograd wrapper for training (the step after the attention hot path).

LLaMA-Factory PR "efficient tuning for gpt-oss", "What I Changed": gpt-oss is
fine-tuned with a fused sink-attention kernel and gradient checkpointing.
This module gives torch's autograd a function over the library's forward and
backward entry points: the forward saves its inputs plus out and lse (O(S)
per head, no S x S matrix), the backward hands them to gptoss_attn_bwd.  It
marshals arguments only; both directions run in the HIP kernels.

    out = sink_attention(q, k, v, sinks, window=128)
    out.backward(dout)   # fills q.grad, k.grad, v.grad, sinks.grad

Under torch.utils.checkpoint the forward simply runs again during the
backward pass (it is deterministic, so the recomputed out/lse are bitwise
the ones of the first pass).
"""

import math

import torch

from . import bwd as _bwd
from . import bwd_rope as _bwd_rope
from . import fwd as _fwd
from . import fwd_rope as _fwd_rope

__all__ = ["SinkAttentionFunction", "sink_attention", "SinkAttentionRopeFunction", "sink_attention_rope"]


class SinkAttentionFunction(torch.autograd.Function):
    """(q, k, v, sinks, window, scale) -> (out, lse); lse is not differentiable."""

    @staticmethod
    def forward(ctx, q, k, v, sinks, window, scale):
        out, lse = _fwd(q, k, v, sinks, window, scale)
        ctx.save_for_backward(q, k, v, sinks, out, lse)
        ctx.window = window
        ctx.scale = scale
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, sinks, out, lse = ctx.saved_tensors
        if dout is None:
            return None, None, None, None, None, None
        dq, dk, dv, dsinks = _bwd(q, k, v, sinks, out, lse, dout.contiguous(), ctx.window, ctx.scale)
        needs = ctx.needs_input_grad
        return (dq if needs[0] else None, dk if needs[1] else None, dv if needs[2] else None,
                dsinks if needs[3] else None, None, None)


def sink_attention(q, k, v, sinks, window=0, scale=None, return_lse=False):
    """Causal (window = 0) or sliding-window grouped-query attention with a
    per-head sink logit; differentiable in q, k, v and sinks.

    q [B, S, Hq, 64], k/v [B, S, Hkv, 64] bf16, sinks [Hq] fp32, all on the
    HIP device and contiguous.  Returns out [B, S, Hq, 64] bf16 (and lse
    [B, Hq, S] fp32 when return_lse)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    out, lse = SinkAttentionFunction.apply(q, k, v, sinks, int(window), float(scale))
    return (out, lse) if return_lse else out


class SinkAttentionRopeFunction(torch.autograd.Function):
    """(q, k, v, sinks, table, window, scale) -> out, with the YaRN rotary
    embedding of q and k fused in (gptoss_attn_fwd_rope / _bwd_rope); saves
    q, the rotated keys, v, sinks, out and lse."""

    @staticmethod
    def forward(ctx, q, k, v, sinks, table, window, scale):
        out, lse, k_rot = _fwd_rope(q, k, v, sinks, table, window, scale)
        ctx.save_for_backward(q, k_rot, v, sinks, table, out, lse)
        ctx.window = window
        ctx.scale = scale
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k_rot, v, sinks, table, out, lse = ctx.saved_tensors
        dq, dk, dv, dsinks = _bwd_rope(q, k_rot, v, sinks, table, out, lse, dout.contiguous(), ctx.window, ctx.scale)
        needs = ctx.needs_input_grad
        return (dq if needs[0] else None, dk if needs[1] else None, dv if needs[2] else None,
                dsinks if needs[3] else None, None, None, None)


def sink_attention_rope(q, k, v, sinks, table, window=0, scale=None):
    """sink_attention over q and k rotated by the rotary table (token i of
    each sequence at position i; table from attention_attn_fwd_amd.rope_table);
    differentiable in the unrotated q, k and in v and sinks."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return SinkAttentionRopeFunction.apply(q, k, v, sinks, table, int(window), float(scale))
