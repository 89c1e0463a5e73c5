"""PyTorch autograd binding of the forward and backward entry points.

``linear_attention(q, k, v, causal)`` returns the attention output and, when a
loss is back-propagated through it, produces dq, dk, dv with
``linattn_backward_after_forward``: the forward's workspace (its per-segment
state records) is kept with the autograd node and reused, so the backward does
not recompute the segment states ("[Paper Review] Transformers are RNNs",
§3.5: the gradients are cumulative sums, linear in time and memory).

Only marshalling happens here; both directions run in the HIP kernels.
Higher-order gradients are not supported.
"""
from __future__ import annotations

import torch

from . import backward, backward_workspace_bytes, forward


class LinearAttentionFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal: bool = True):
        B, H, N, _ = q.shape
        ws = torch.empty(backward_workspace_bytes(B, H, N, q.dtype, causal), dtype=torch.uint8, device=q.device)
        o = forward(q, k, v, causal=causal, workspace=ws)
        ctx.save_for_backward(q, k, v)
        ctx.workspace = ws
        ctx.causal = causal
        return o

    @staticmethod
    def backward(ctx, grad_o):
        # The backward only reads the forward's records (it writes its own
        # part of the workspace), so a retained graph can be back-propagated
        # again; saved-tensor version checks catch in-place changes of q, k, v.
        q, k, v = ctx.saved_tensors
        g = grad_o.to(v.dtype).contiguous()
        dq, dk, dv = backward(q, k, v, g, causal=ctx.causal, workspace=ctx.workspace, after_forward=True)
        return dq, dk, dv, None


def linear_attention(q, k, v, causal: bool = True):
    """Linear attention with phi = elu + 1 and autograd support.

    q, k: [B, H, N, 64]; v: [B, H, N, 64]; float32 or bfloat16, contiguous, on a GPU.
    Returns o [B, H, N, 64] in the input dtype."""
    return LinearAttentionFunction.apply(q, k, v, causal)
