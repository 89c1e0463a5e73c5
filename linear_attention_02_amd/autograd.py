"""PyTorch autograd binding of the training entry points.

``linear_attention(q, k, v, causal)`` returns the attention output through
``linattn_forward_train``, which also saves what the backward needs (the
segment state records and 1/den per token) in a workspace kept with the
autograd node.  Back-propagating a loss through it runs
``linattn_backward_train`` on that workspace and the saved output: for
causal bf16 inputs one pass forms the reverse sums from Q, dO and O and one
left-to-right pass writes dq, dk and dv ("[Paper Review] Transformers are
RNNs", §3.5: the gradients are cumulative sums, linear in time and memory);
other inputs take the backward that reuses the forward's records.

Only marshalling happens here; both directions run in the HIP kernels.
Higher-order gradients are not supported.
"""
from __future__ import annotations

import torch

from . import backward_train, forward_train


class LinearAttentionFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal: bool = True):
        o, ws = forward_train(q, k, v, causal=causal)
        ctx.save_for_backward(q, k, v, o)
        ctx.workspace = ws
        ctx.causal = causal
        return o

    @staticmethod
    def backward(ctx, grad_o):
        # The backward only reads what the forward saved (it writes its own
        # part of the workspace), so a retained graph can be back-propagated
        # again; saved-tensor version checks catch in-place changes of q, k,
        # v and o.
        q, k, v, o = ctx.saved_tensors
        g = grad_o.to(v.dtype).contiguous()
        dq, dk, dv = backward_train(q, k, v, o, g, ctx.workspace, causal=ctx.causal)
        return dq, dk, dv, None


def linear_attention(q, k, v, causal: bool = True):
    """Linear attention with phi = elu + 1 and autograd support.

    q, k: [B, H, N, 64]; v: [B, H, N, 64]; float32 or bfloat16, contiguous, on a GPU.
    Returns o [B, H, N, 64] in the input dtype."""
    return LinearAttentionFunction.apply(q, k, v, causal)
