"""torch.autograd wrapper around ``flce_fwd_bwd``.

All gradients come out of the forward call (PR #1554, Summary: the logits,
grad_input and grad_weight GEMMs all run inside the forward).  Backward only
scales them by the upstream gradient; for ``reduction="none"`` the upstream
gradient is per token and unknown at forward time, so backward calls the
library again with it (PR #1554, Tests: the none reduction re-enters the chunk
loop with reusable buffers).  The fp32 -> weight-dtype cast of grad_weight
and the upstream scaling run in the library's scale/cast kernel.
"""
from __future__ import annotations

import torch

from . import fused_linear_cross_entropy_fwd_bwd, scale_cast


class FusedLinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, target, ignore_index, reduction, chunk_size, chunk_mem_const,
                accum_dtype, frozen_weight):
        frozen = bool(frozen_weight) or not weight.requires_grad
        ctx.cfg = (ignore_index, reduction, chunk_size, chunk_mem_const, accum_dtype, frozen)
        r = fused_linear_cross_entropy_fwd_bwd(
            x, weight, target, ignore_index=ignore_index, reduction=reduction,
            chunk_size=chunk_size, chunk_mem_const=chunk_mem_const, accum_dtype=accum_dtype,
            frozen_weight=frozen)
        if reduction == "none":
            ctx.save_for_backward(x, weight, target)
        else:
            ctx.save_for_backward(r.dX, r.dW if r.dW is not None else torch.empty(0))
        return r.loss

    @staticmethod
    def backward(ctx, grad_loss):
        ignore_index, reduction, chunk_size, chunk_mem_const, accum_dtype, frozen = ctx.cfg
        if reduction == "none":
            x, weight, target = ctx.saved_tensors
            r = fused_linear_cross_entropy_fwd_bwd(
                x, weight, target, ignore_index=ignore_index, reduction="none",
                chunk_size=chunk_size, chunk_mem_const=chunk_mem_const, accum_dtype=accum_dtype,
                frozen_weight=frozen, grad_output=grad_loss.float())
            dX, dW = r.dX, r.dW
            if dW is not None and dW.dtype != weight.dtype:
                dW = scale_cast(dW, weight.dtype)
            return dX, dW, None, None, None, None, None, None, None
        dX, dW = ctx.saved_tensors
        g = grad_loss.reshape(1).float()
        dX = scale_cast(dX, dX.dtype, scale=g, out=dX)
        if frozen:
            dW = None
        else:
            wdt = dX.dtype
            dW = scale_cast(dW, wdt, scale=g, out=dW if dW.dtype == wdt else None)
        return dX, dW, None, None, None, None, None, None, None


def fused_linear_cross_entropy(x, weight, target, *, ignore_index: int = -100,
                               reduction: str = "mean", chunk_size: int | None = None,
                               chunk_mem_const: int = 1, accum_dtype=None,
                               frozen_weight: bool | None = None):
    """Loss of lm_head projection + cross-entropy, differentiable w.r.t. x and weight.

    ``accum_dtype=torch.float32`` accumulates grad_weight in fp32 and casts it
    to the weight dtype at the end; None accumulates in the weight dtype.
    """
    return FusedLinearCrossEntropy.apply(x, weight, target, ignore_index, reduction, chunk_size,
                                         chunk_mem_const, accum_dtype, bool(frozen_weight))
