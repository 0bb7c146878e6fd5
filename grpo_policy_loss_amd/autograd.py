"""torch.autograd wrapper over the C ABI: the loss as a differentiable function of
the hidden states H and the LM head W, for use inside a PyTorch training step.

The forward is grpo_loss_fwd; the backward is grpo_loss_bwd with the upstream
gradient of the loss as its grad_loss (Unsloth docs, "Offloading activations
for log softmax": the backward recomputes the chunk's logits instead of
keeping them).  Marshalling only: both passes run in libgrpo.so.
"""
from __future__ import annotations

import torch

from ._lib import grpo_loss_bwd, grpo_loss_fwd


class _GrpoLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, y, mask, adv, ref_lp, B, L, beta, chunk, opts):
        loss, lp, kl, lse = grpo_loss_fwd(H, W, y, mask, adv, ref_lp, B, L, beta, chunk,
                                          opts=opts)
        ctx.save_for_backward(H, W, y, mask, adv, ref_lp, lp, lse)
        ctx.args = (B, L, beta, chunk, opts)
        ctx.mark_non_differentiable(lp, kl)
        return loss.reshape(()), lp, kl

    @staticmethod
    def backward(ctx, g_loss, g_lp, g_kl):
        H, W, y, mask, adv, ref_lp, lp, lse = ctx.saved_tensors
        B, L, beta, chunk, opts = ctx.args
        # the C ABI takes the upstream scalar by value: one host read of it
        g = 0.0 if g_loss is None else float(g_loss)
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_h or need_w) or g == 0.0:
            return (torch.zeros_like(H) if need_h else None,
                    torch.zeros_like(W) if need_w else None) + (None,) * 9
        dH, dW = grpo_loss_bwd(H, W, y, mask, adv, ref_lp, lp, lse, B, L, beta, g, chunk,
                               opts=opts)
        return (dH if need_h else None,
                (dW if W.dtype == torch.float32 else dW.to(W.dtype)) if need_w else None) \
            + (None,) * 9


def grpo_loss(H, W, y, mask, adv, ref_lp, B: int, L: int, beta: float = 0.04,
              chunk: int = 4096, opts=None):
    """(loss, lp, kl): loss is a 0-d float32 tensor differentiable with respect to H
    and W; lp and kl ([N] float32) carry no gradient.  Arguments as for
    grpo_loss_fwd.  W's gradient is formed in float32 and returned in W's dtype: a
    bfloat16 W receives it rounded to bfloat16 (grpo_loss_bwd with a float32 dW
    accumulator keeps it in float32).  The backward reads the upstream gradient of
    the loss on the host (one synchronisation)."""
    return _GrpoLoss.apply(H, W, y, mask, adv, ref_lp, B, L, beta, chunk, opts)
