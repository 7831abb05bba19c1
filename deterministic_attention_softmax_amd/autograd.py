"""An autograd Function over jas_fwd / jas_bwd (argument marshalling only:
both directions are the library's kernels).

RL-Kernel PR #453, Fixed-order backward: the backward reads the stored P
and dP and returns dScores; ROCm TransformerEngine PR #678, Description:
the sink's gradient comes out of the same backward.  RL-Kernel PR #240's
review of its autograd wrapper: the tensors the backward needs are saved
with save_for_backward, and the backward, an opaque library call with no
autograd graph of its own, is once-differentiable, so a request for a
second derivative fails with an explicit error.

The additive mask and the key lengths are constants (no gradient); the
sink probability is returned as a non-differentiable output.  The scores
are made contiguous, so P and the incoming dP share one row layout.
"""
import torch
from torch.autograd.function import once_differentiable

from . import bwd as _bwd
from . import fwd as _fwd


class JasSoftmax(torch.autograd.Function):
    @staticmethod
    def forward(ctx, scores, sink, mask, mask_strides, causal, key_len):
        P, p_sink = _fwd(scores.contiguous(), mask=mask, mask_strides=mask_strides, sink=sink,
                         causal=causal, key_len=key_len)
        saved = [P]
        if sink is not None:
            saved.append(p_sink)
        if key_len is not None:
            saved.append(key_len)
        ctx.save_for_backward(*saved)
        ctx.has_sink = sink is not None
        ctx.has_key_len = key_len is not None
        ctx.causal = bool(causal)
        if p_sink is None:
            return P
        ctx.mark_non_differentiable(p_sink)
        return P, p_sink

    @staticmethod
    @once_differentiable
    def backward(ctx, dP, *unused):
        saved = list(ctx.saved_tensors)
        P = saved.pop(0)
        p_sink = saved.pop(0) if ctx.has_sink else None
        key_len = saved.pop(0) if ctx.has_key_len else None
        dS, d_sink = _bwd(P, dP.to(P.dtype).contiguous(), p_sink=p_sink, causal=ctx.causal,
                          key_len=key_len)
        return dS, d_sink, None, None, None, None


def softmax(scores, sink=None, mask=None, mask_strides=None, causal=False, key_len=None):
    """P = the fixed-order row softmax of ``scores`` [B, H, Sq, N] (with the
    sink in the denominator when ``sink`` fp32 [H] is given), differentiable
    in the scores and the sink.  Returns P, or (P, p_sink) with a sink."""
    return JasSoftmax.apply(scores, sink, mask, mask_strides, causal, key_len)
