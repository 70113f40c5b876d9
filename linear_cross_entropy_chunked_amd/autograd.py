"""torch.autograd wrapper around ``flce_fwd_bwd_ex``.

For mean and sum every gradient comes out of the forward call (PR #1554,
Summary: the logits, grad_input and grad_weight GEMMs all run inside the
forward); backward only scales them by the upstream gradient.  For
``reduction="none"`` the upstream gradient is per token and unknown at
forward time, so the forward asks the library for the loss only (no logits
slab, no gradient GEMMs) and backward calls it again with that gradient
(PR #1554, Tests: the none reduction re-enters the chunk loop with reusable
buffers).  The fp32 -> weight-dtype cast of grad_weight and grad_bias and the
upstream scaling run in the library's scale/cast kernel.
"""
from __future__ import annotations

import torch

from . import fused_linear_cross_entropy_fwd_bwd, scale_cast


def _grads_to(dtype, g, tensors, owned: bool):
    """Scale each fp32-or-native gradient by the device scalar g (None = 1) into dtype.

    ``owned`` says the tensors are this backward's own (fresh from a library
    call), so one already in ``dtype`` with no scale is returned as it is.
    Tensors saved by the forward are never written: a second backward through
    a retained graph must see them unchanged, and the returned gradient must
    not share storage with them.
    """
    out = []
    for t in tensors:
        if t is None:
            out.append(None)
        elif owned and g is None and t.dtype == dtype:
            out.append(t)
        else:
            out.append(scale_cast(t, dtype, scale=g))
    return out


class FusedLinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, target, bias, ignore_index, reduction, chunk_size,
                chunk_mem_const, accum_dtype, frozen_weight, z_loss_scale):
        frozen = bool(frozen_weight) or not weight.requires_grad
        need_grads = x.requires_grad or not frozen or (bias is not None and bias.requires_grad)
        ctx.cfg = (ignore_index, reduction, chunk_size, chunk_mem_const, accum_dtype, frozen,
                   z_loss_scale, bias is not None)
        kw = dict(bias=bias, ignore_index=ignore_index, reduction=reduction,
                  chunk_size=chunk_size, chunk_mem_const=chunk_mem_const,
                  accum_dtype=accum_dtype, frozen_weight=frozen, z_loss_scale=z_loss_scale)
        if reduction == "none" or not need_grads:
            r = fused_linear_cross_entropy_fwd_bwd(x, weight, target, forward_only=True, **kw)
            ctx.save_for_backward(x, weight, target, bias)
            ctx.deferred = True
        else:
            r = fused_linear_cross_entropy_fwd_bwd(x, weight, target, **kw)
            empty = torch.empty(0, device=x.device)
            ctx.save_for_backward(r.dX, r.dW if r.dW is not None else empty,
                                  r.grad_bias if r.grad_bias is not None else empty)
            ctx.deferred = False
        return r.loss

    @staticmethod
    def backward(ctx, grad_loss):
        (ignore_index, reduction, chunk_size, chunk_mem_const, accum_dtype, frozen, z_loss_scale,
         has_bias) = ctx.cfg
        if ctx.deferred:
            x, weight, target, bias = ctx.saved_tensors
            go = grad_loss.float().reshape(-1)
            r = fused_linear_cross_entropy_fwd_bwd(
                x, weight, target, bias=bias, ignore_index=ignore_index, reduction=reduction,
                chunk_size=chunk_size, chunk_mem_const=chunk_mem_const, accum_dtype=accum_dtype,
                frozen_weight=frozen, z_loss_scale=z_loss_scale, grad_output=go)
            dX, dW, db = r.dX, r.dW, r.grad_bias
            dW, db = _grads_to(weight.dtype, None, [dW, db], owned=True)
        else:
            dX, dW, db = ctx.saved_tensors
            g = grad_loss.reshape(1).float()
            dW = None if frozen else dW
            db = db if has_bias else None
            dX, dW, db = _grads_to(dX.dtype, g, [dX, dW, db], owned=False)
        return dX, dW, None, db, None, None, None, None, None, None, None


def fused_linear_cross_entropy(x, weight, target, bias=None, *, ignore_index: int = -100,
                               reduction: str = "mean", chunk_size: int | None = None,
                               chunk_mem_const: int = 1, accum_dtype=None,
                               frozen_weight: bool | None = None, z_loss_scale: float = 0.0):
    """Loss of the lm_head projection (+ bias) followed by cross-entropy,
    differentiable with respect to x, weight and bias.

    ``accum_dtype=torch.float32`` accumulates grad_weight and grad_bias in
    fp32 and casts them to the weight dtype at the end; None accumulates in
    the weight dtype.  ``z_loss_scale`` adds lam * logsumexp(z)^2 per
    labelled row.
    """
    return FusedLinearCrossEntropy.apply(x, weight, target, bias, ignore_index, reduction,
                                         chunk_size, chunk_mem_const, accum_dtype,
                                         bool(frozen_weight), float(z_loss_scale))
