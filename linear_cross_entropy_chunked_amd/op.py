"""Fused linear cross-entropy as a torch custom op (``torch.ops.flce.*``).

Registered with torch.library so that torch.compile treats the whole call as
one opaque node instead of tracing into it (PR #1554, Details item 6 and
Summary: under torch.compile the library path must give the same results as
eager).  Two ops, each with a fake (shape-only) implementation for tracing:

  flce::fused_linear_cross_entropy(x, weight, target, bias, ...)
      -> (loss, grad_x, grad_weight, grad_bias)
      mean / sum: the gradients come out of the same call, for an upstream
      gradient of 1; none: loss only (the gradients are empty).
  flce::fused_linear_cross_entropy_backward(x, weight, target, bias,
                                            grad_loss, ...)
      -> (grad_x, grad_weight, grad_bias)
      the none reduction's backward: the chunk loop again, with the per-token
      upstream gradient.

``fused_linear_cross_entropy_op`` is the differentiable entry (autograd is
registered on the first op); it returns the loss.  A third op,
flce::scale_cast, applies the upstream gradient in backward with the
library's scale/cast kernel, so that a compiled backward stays traceable.  The
ops run the HIP library; they have no CPU implementation.
"""

from typing import Optional

import torch
from torch import Tensor

from . import fused_linear_cross_entropy_fwd_bwd, scale_cast


def _accum(x: Tensor, accum_fp32: bool):
    return torch.float32 if accum_fp32 else x.dtype


@torch.library.custom_op("flce::fused_linear_cross_entropy", mutates_args=())
def _fwd(x: Tensor, weight: Tensor, target: Tensor, bias: Optional[Tensor], ignore_index: int,
         reduction: str, chunk_size: int, chunk_mem_const: int, accum_fp32: bool,
         frozen_weight: bool, z_loss_scale: float, need_grads: bool
         ) -> tuple[Tensor, Tensor, Tensor, Tensor]:
    loss_only = reduction == "none" or not need_grads
    r = fused_linear_cross_entropy_fwd_bwd(
        x, weight, target, bias=bias, ignore_index=ignore_index, reduction=reduction,
        chunk_size=chunk_size or None, chunk_mem_const=chunk_mem_const,
        accum_dtype=torch.float32 if accum_fp32 else None, frozen_weight=frozen_weight,
        z_loss_scale=z_loss_scale, forward_only=loss_only)
    loss = r.loss if reduction == "none" else r.loss.reshape(())
    dX = r.dX if r.dX is not None else x.new_empty(0)
    dW = r.dW if r.dW is not None else x.new_empty(0)
    db = r.grad_bias if r.grad_bias is not None else x.new_empty(0)
    return loss, dX, dW, db


@_fwd.register_fake
def _fwd_fake(x, weight, target, bias, ignore_index, reduction, chunk_size, chunk_mem_const,
              accum_fp32, frozen_weight, z_loss_scale, need_grads):
    BT = x.shape[0]
    loss = x.new_empty((BT,) if reduction == "none" else (), dtype=torch.float32)
    if reduction == "none" or not need_grads:
        return loss, x.new_empty(0), x.new_empty(0), x.new_empty(0)
    adt = _accum(x, accum_fp32)
    dW = x.new_empty(0) if frozen_weight else weight.new_empty(weight.shape, dtype=adt)
    db = x.new_empty(0) if bias is None else weight.new_empty((weight.shape[0],), dtype=adt)
    return loss, torch.empty_like(x), dW, db


@torch.library.custom_op("flce::fused_linear_cross_entropy_backward", mutates_args=())
def _bwd(x: Tensor, weight: Tensor, target: Tensor, bias: Optional[Tensor], grad_loss: Tensor,
         ignore_index: int, reduction: str, chunk_size: int, chunk_mem_const: int,
         accum_fp32: bool, frozen_weight: bool, z_loss_scale: float
         ) -> tuple[Tensor, Tensor, Tensor]:
    r = fused_linear_cross_entropy_fwd_bwd(
        x, weight, target, bias=bias, ignore_index=ignore_index, reduction=reduction,
        chunk_size=chunk_size or None, chunk_mem_const=chunk_mem_const,
        accum_dtype=torch.float32 if accum_fp32 else None, frozen_weight=frozen_weight,
        z_loss_scale=z_loss_scale, grad_output=grad_loss.float().reshape(-1))
    dW = r.dW if r.dW is not None else x.new_empty(0)
    db = r.grad_bias if r.grad_bias is not None else x.new_empty(0)
    return r.dX, dW, db


@_bwd.register_fake
def _bwd_fake(x, weight, target, bias, grad_loss, ignore_index, reduction, chunk_size,
              chunk_mem_const, accum_fp32, frozen_weight, z_loss_scale):
    adt = _accum(x, accum_fp32)
    dW = x.new_empty(0) if frozen_weight else weight.new_empty(weight.shape, dtype=adt)
    db = x.new_empty(0) if bias is None else weight.new_empty((weight.shape[0],), dtype=adt)
    return torch.empty_like(x), dW, db


@torch.library.custom_op("flce::scale_cast", mutates_args=())
def _scale_cast(src: Tensor, dtype: torch.dtype, scale: Optional[Tensor]) -> Tensor:
    """scale * src converted to dtype, by the library's scale/cast kernel."""
    return scale_cast(src, dtype, scale=scale)


@_scale_cast.register_fake
def _scale_cast_fake(src, dtype, scale):
    return src.new_empty(src.shape, dtype=dtype)


def _setup_context(ctx, inputs, output):
    (x, weight, target, bias, ignore_index, reduction, chunk_size, chunk_mem_const, accum_fp32,
     frozen_weight, z_loss_scale, need_grads) = inputs
    _, dX, dW, db = output
    ctx.cfg = (ignore_index, reduction, chunk_size, chunk_mem_const, accum_fp32, frozen_weight,
               z_loss_scale, bias is not None, weight.dtype)
    if reduction == "none":
        ctx.save_for_backward(x, weight, target, bias)
    else:
        ctx.save_for_backward(dX, dW, db)


def _cast_scaled(t: Tensor, dtype, g: Optional[Tensor]):
    if t.numel() == 0:
        return None
    if g is None and t.dtype == dtype:
        return t
    return torch.ops.flce.scale_cast(t, dtype, g)


def _backward(ctx, grad_loss, _gx, _gw, _gb):
    (ignore_index, reduction, chunk_size, chunk_mem_const, accum_fp32, frozen_weight,
     z_loss_scale, has_bias, wdt) = ctx.cfg
    if reduction == "none":
        x, weight, target, bias = ctx.saved_tensors
        dX, dW, db = torch.ops.flce.fused_linear_cross_entropy_backward(
            x, weight, target, bias, grad_loss, ignore_index, reduction, chunk_size,
            chunk_mem_const, accum_fp32, frozen_weight, z_loss_scale)
        g = None
    else:
        dX, dW, db = ctx.saved_tensors
        g = grad_loss.reshape(1).float()
    gx = _cast_scaled(dX, dX.dtype, g)
    gw = None if frozen_weight else _cast_scaled(dW, wdt, g)
    gb = _cast_scaled(db, wdt, g) if has_bias else None
    return gx, gw, None, gb, None, None, None, None, None, None, None, None


torch.library.register_autograd("flce::fused_linear_cross_entropy", _backward,
                                setup_context=_setup_context)


def fused_linear_cross_entropy_op(x: Tensor, weight: Tensor, target: Tensor,
                                  bias: Optional[Tensor] = None, *, ignore_index: int = -100,
                                  reduction: str = "mean", chunk_size: int = 0,
                                  chunk_mem_const: int = 1, accum_fp32: bool = False,
                                  frozen_weight: bool = False, z_loss_scale: float = 0.0) -> Tensor:
    """Differentiable fused linear cross-entropy through ``torch.ops.flce``."""
    need = bool(x.requires_grad or (weight.requires_grad and not frozen_weight)
                or (bias is not None and bias.requires_grad))
    frozen = bool(frozen_weight or not weight.requires_grad)
    loss, _, _, _ = torch.ops.flce.fused_linear_cross_entropy(
        x, weight, target, bias, ignore_index, reduction, int(chunk_size), int(chunk_mem_const),
        bool(accum_fp32), frozen, float(z_loss_scale), need)
    return loss
