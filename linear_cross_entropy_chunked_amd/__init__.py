"""Fused linear cross-entropy on MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in ``include/flce.h`` (``libflce.so``,
built from ``csrc/`` by ``build.py``).  The functions named ``flce_*`` take
the same arguments as the C entry points (device pointers as ints); the
convenience wrappers below only allocate outputs and workspace with torch and
marshal pointers.  Every step of the computation runs in the HIP kernels:
there is no fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflce.so")

F32, F16, BF16 = 0, 1, 2
SCRATCH_BYTES = 256 << 20  # FLCE_SCRATCH_BYTES: the static workspace of flce_fwd_bwd_ex_noalloc
MEAN, SUM, NONE = 0, 1, 2
REDUCTIONS = {"mean": MEAN, "sum": SUM, "none": NONE}
STATUS = {0: "FLCE_OK", -1: "FLCE_E_ARG", -2: "FLCE_E_DTYPE", -3: "FLCE_E_TARGET",
          -4: "FLCE_E_WORKSPACE", -5: "FLCE_E_HIP"}
KERNEL_KINDS = ["mask_scan", "zero_ignored_rows", "logits_gemm", "softmax_grad", "dx_gemm",
                "dx_reduce", "dw_gemm", "loss_finalize", "fill_cast", "gather_rows",
                "bias_grad"]

# Every symbol include/flce.h declares.
EXPORTS = ["flce_chunk_size", "flce_chunk_size_mi355x", "flce_workspace_bytes", "flce_fwd_bwd",
           "flce_workspace_bytes_ex", "flce_workspace_row_index_offset", "flce_fwd_bwd_ex",
           "flce_fwd_bwd_ex_noalloc", "flce_scale_cast", "flce_status_string", "flce_last_error",
           "flce_profile_begin", "flce_profile_begin_kinds", "flce_profile_end",
           "flce_kernel_name"]


class FlceError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = ""
        if status == -5:
            detail = ": " + flce_last_error()
        super().__init__(f"{where} failed with {STATUS.get(status, status)}{detail}")


class FlceStats(ctypes.Structure):
    _fields_ = [("chunk_size", ctypes.c_int64), ("chunks_total", ctypes.c_int64),
                ("chunks_run", ctypes.c_int64), ("n_valid", ctypes.c_int64),
                ("compacted", ctypes.c_int32), ("dx_splits", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class FlceProfile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 11), ("total_ms", ctypes.c_double * 11)]


class FlceOptions(ctypes.Structure):
    """flce_options_t: the optional parts of the method (device pointers as ints)."""
    _fields_ = [("forward_only", ctypes.c_int32), ("bias", ctypes.c_void_p),
                ("grad_bias", ctypes.c_void_p), ("z_loss_scale", ctypes.c_float),
                ("z_loss", ctypes.c_void_p), ("accuracy", ctypes.c_void_p),
                ("predicted", ctypes.c_void_p)]


_lib = None


def load():
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    I = ctypes.c_int
    lib.flce_chunk_size.argtypes = [I64, I64, I64, I64, I32]
    lib.flce_chunk_size.restype = I64
    lib.flce_chunk_size_mi355x.argtypes = [I64, I64, I64, I, I, I32, SZ]
    lib.flce_chunk_size_mi355x.restype = I64
    lib.flce_workspace_bytes.argtypes = [I64, I64, I64, I, I64, I32]
    lib.flce_workspace_bytes.restype = SZ
    lib.flce_fwd_bwd.argtypes = [P, P, P, I64, I64, I64, I, I64, I, I64, I32, I, I32, I32, P, P,
                                 P, P, P, SZ, P, ctypes.POINTER(FlceStats)]
    lib.flce_fwd_bwd.restype = I
    lib.flce_workspace_bytes_ex.argtypes = [I64, I64, I64, I, I64, I32,
                                            ctypes.POINTER(FlceOptions)]
    lib.flce_workspace_bytes_ex.restype = SZ
    lib.flce_workspace_row_index_offset.argtypes = [I64, I64, I64, I, I64, I32,
                                                    ctypes.POINTER(FlceOptions)]
    lib.flce_workspace_row_index_offset.restype = SZ
    lib.flce_fwd_bwd_ex.argtypes = [P, P, P, I64, I64, I64, I, I64, I, I64, I32, I, I32, I32, P,
                                    P, P, P, P, SZ, P, ctypes.POINTER(FlceStats),
                                    ctypes.POINTER(FlceOptions)]
    lib.flce_fwd_bwd_ex.restype = I
    lib.flce_fwd_bwd_ex_noalloc.argtypes = [P, P, P, I64, I64, I64, I, I64, I, I64, I32, I, I32,
                                            I32, P, P, P, P, P, ctypes.POINTER(FlceStats),
                                            ctypes.POINTER(FlceOptions)]
    lib.flce_fwd_bwd_ex_noalloc.restype = I
    lib.flce_scale_cast.argtypes = [P, I, P, I, I64, P, P]
    lib.flce_scale_cast.restype = I
    lib.flce_status_string.argtypes = [I]
    lib.flce_status_string.restype = ctypes.c_char_p
    lib.flce_last_error.argtypes = []
    lib.flce_last_error.restype = ctypes.c_char_p
    lib.flce_profile_begin.argtypes = []
    lib.flce_profile_begin.restype = I
    lib.flce_profile_begin_kinds.argtypes = [ctypes.c_uint32]
    lib.flce_profile_begin_kinds.restype = I
    lib.flce_profile_end.argtypes = [ctypes.POINTER(FlceProfile)]
    lib.flce_profile_end.restype = I
    lib.flce_kernel_name.argtypes = [I]
    lib.flce_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ----------------------------------------------------------- C-ABI mirrors
def flce_chunk_size(BT: int, H: int, V: int, chunk_size: int = 0, chunk_mem_const: int = 1) -> int:
    return load().flce_chunk_size(BT, H, V, chunk_size, chunk_mem_const)


def flce_chunk_size_mi355x(BT: int, H: int, V: int, dtype: int, accum_dtype: int,
                           frozen_weight: int = 0, slab_budget_bytes: int = 0) -> int:
    return load().flce_chunk_size_mi355x(BT, H, V, dtype, accum_dtype, frozen_weight,
                                         slab_budget_bytes)


def flce_workspace_bytes(BT: int, H: int, V: int, dtype: int, chunk_size: int = 0,
                         chunk_mem_const: int = 1) -> int:
    return load().flce_workspace_bytes(BT, H, V, dtype, chunk_size, chunk_mem_const)


def flce_fwd_bwd(X: int, W: int, targets: int, BT: int, H: int, V: int, dtype: int,
                 ignore_index: int, reduction: int, chunk_size: int, chunk_mem_const: int,
                 accum_dtype: int, frozen_weight: int, accumulate_dw: int, grad_output,
                 loss: int, dX: int, dW, workspace: int, workspace_bytes: int, stream,
                 stats: FlceStats | None = None) -> int:
    return load().flce_fwd_bwd(X, W, targets, BT, H, V, dtype, ignore_index, reduction,
                               chunk_size, chunk_mem_const, accum_dtype, frozen_weight,
                               accumulate_dw, grad_output, loss, dX, dW, workspace,
                               workspace_bytes, stream,
                               ctypes.byref(stats) if stats is not None else None)


def flce_workspace_bytes_ex(BT: int, H: int, V: int, dtype: int, chunk_size: int = 0,
                            chunk_mem_const: int = 1, opt: FlceOptions | None = None) -> int:
    return load().flce_workspace_bytes_ex(BT, H, V, dtype, chunk_size, chunk_mem_const,
                                          ctypes.byref(opt) if opt is not None else None)


def flce_workspace_row_index_offset(BT: int, H: int, V: int, dtype: int, chunk_size: int = 0,
                                    chunk_mem_const: int = 1,
                                    opt: FlceOptions | None = None) -> int:
    return load().flce_workspace_row_index_offset(
        BT, H, V, dtype, chunk_size, chunk_mem_const,
        ctypes.byref(opt) if opt is not None else None)


def flce_fwd_bwd_ex(X: int, W: int, targets: int, BT: int, H: int, V: int, dtype: int,
                    ignore_index: int, reduction: int, chunk_size: int, chunk_mem_const: int,
                    accum_dtype: int, frozen_weight: int, accumulate_dw: int, grad_output,
                    loss: int, dX, dW, workspace: int, workspace_bytes: int, stream,
                    stats: FlceStats | None = None, opt: FlceOptions | None = None) -> int:
    return load().flce_fwd_bwd_ex(X, W, targets, BT, H, V, dtype, ignore_index, reduction,
                                  chunk_size, chunk_mem_const, accum_dtype, frozen_weight,
                                  accumulate_dw, grad_output, loss, dX, dW, workspace,
                                  workspace_bytes, stream,
                                  ctypes.byref(stats) if stats is not None else None,
                                  ctypes.byref(opt) if opt is not None else None)


def flce_fwd_bwd_ex_noalloc(X: int, W: int, targets: int, BT: int, H: int, V: int, dtype: int,
                            ignore_index: int, reduction: int, chunk_size: int,
                            chunk_mem_const: int, accum_dtype: int, frozen_weight: int,
                            accumulate_dw: int, grad_output, loss: int, dX, dW, stream,
                            stats: FlceStats | None = None, opt: FlceOptions | None = None) -> int:
    return load().flce_fwd_bwd_ex_noalloc(X, W, targets, BT, H, V, dtype, ignore_index, reduction,
                                          chunk_size, chunk_mem_const, accum_dtype,
                                          frozen_weight, accumulate_dw, grad_output, loss, dX, dW,
                                          stream,
                                          ctypes.byref(stats) if stats is not None else None,
                                          ctypes.byref(opt) if opt is not None else None)


def flce_scale_cast(src: int, src_dtype: int, dst: int, dst_dtype: int, n: int, scale,
                    stream) -> int:
    return load().flce_scale_cast(src, src_dtype, dst, dst_dtype, n, scale, stream)


def flce_status_string(status: int) -> str:
    return load().flce_status_string(status).decode()


def flce_last_error() -> str:
    return load().flce_last_error().decode()


def flce_profile_begin() -> int:
    return load().flce_profile_begin()


def flce_profile_begin_kinds(kinds) -> int:
    """Profile only the named kernel kinds (names from KERNEL_KINDS)."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS.index(k)
    return load().flce_profile_begin_kinds(mask)


def flce_profile_end() -> dict:
    p = FlceProfile()
    rc = load().flce_profile_end(ctypes.byref(p))
    if rc != 0:
        raise FlceError(rc, "flce_profile_end")
    return {KERNEL_KINDS[k]: (int(p.launches[k]), float(p.total_ms[k]))
            for k in range(len(KERNEL_KINDS))}


def flce_kernel_name(kind: int) -> str:
    return load().flce_kernel_name(kind).decode()


# ------------------------------------------------------- torch convenience
def _dtype_code(dt) -> int:
    import torch
    m = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if dt not in m:
        raise TypeError(f"unsupported dtype {dt}")
    return m[dt]


def _torch_dtype(code: int):
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[code]


@dataclass
class FlceResult:
    loss: "object"
    dX: "object"
    dW: "object"
    stats: dict
    grad_bias: "object" = None
    z_loss: "object" = None
    accuracy: "object" = None
    predicted: "object" = None
    row_index: "object" = None


def fused_linear_cross_entropy_fwd_bwd(x, weight, target, *, bias=None, ignore_index: int = -100,
                                       reduction: str = "mean", chunk_size: int | None = None,
                                       chunk_mem_const: int = 1, accum_dtype=None,
                                       frozen_weight: bool = False, grad_output=None,
                                       dW=None, accumulate_dw: bool = False,
                                       forward_only: bool = False, z_loss_scale: float = 0.0,
                                       return_z_loss: bool = False,
                                       return_accuracy: bool = False,
                                       return_predicted: bool = False, grad_bias=None,
                                       workspace=None, stream=None,
                                       return_row_index: bool = False) -> FlceResult:
    """Loss, dX and dW (and optionally grad_bias and per-token outputs) in one call.

    x [BT, H], weight [V, H] (float32, float16 or bfloat16, on the GPU),
    target [BT] int64, bias [V] (weight dtype) or None.  ``accum_dtype`` None
    means the weight dtype; pass torch.float32 for fp32 grad_weight and
    grad_bias.  ``dW`` / ``grad_bias`` may be given to write into (and with
    ``accumulate_dw`` to add to).  ``grad_output``: None, a one-element
    float32 tensor (mean/sum) or [BT] float32 (none).  ``chunk_size``: None
    for the pages' heuristic, an int (floored to a power of two, clamped to
    BT), or "mi355x" (or -1) for the MI355X policy.  ``forward_only``
    computes the loss (and the requested per-token outputs) only.
    ``z_loss_scale`` adds lam * lse^2 to every labelled row's loss.
    ``return_row_index`` returns the call's ascending labelled-row index
    (int32 [n_valid]) as a view of the workspace.
    """
    import torch
    if not (x.is_cuda and weight.is_cuda and target.is_cuda):
        raise ValueError("x, weight and target must be on the GPU")
    x = x.contiguous()
    weight = weight.contiguous()
    target = target.contiguous()
    if target.dtype != torch.int64:
        raise TypeError("target must be int64")
    BT, H = x.shape
    V = weight.shape[0]
    dt = _dtype_code(x.dtype)
    if weight.dtype != x.dtype:
        raise TypeError("x and weight must share a dtype")
    if bias is not None:
        if bias.dtype != x.dtype or bias.shape != (V,) or not bias.is_cuda:
            raise TypeError("bias must be a [V] GPU tensor of the weight dtype")
        bias = bias.contiguous()
    adt = dt if accum_dtype is None else _dtype_code(accum_dtype)
    red = REDUCTIONS[reduction]
    if chunk_size in ("mi355x", -1):  # the MI355X default policy
        c = flce_chunk_size_mi355x(BT, H, V, dt, adt, int(bool(frozen_weight)), 0)
        # c is a power of two, or BT when one chunk covers every row; as an
        # explicit size (floored to a power of two, then clamped to BT) its
        # next power of two gives exactly c rows
        cs = 1 << max(int(c) - 1, 0).bit_length() if c > 0 else 0
    else:
        cs = 0 if chunk_size is None else int(chunk_size)
    dev = x.device
    loss = torch.empty(BT if red == NONE else 1, dtype=torch.float32, device=dev)
    nout = BT if red == NONE else 1
    dX = None if forward_only else torch.empty_like(x)
    if forward_only:
        dW = None
    elif not frozen_weight and dW is None:
        dW = torch.empty(V, H, dtype=_torch_dtype(adt), device=dev)
    if bias is not None and not forward_only and grad_bias is None:
        grad_bias = torch.empty(V, dtype=_torch_dtype(adt), device=dev)
    if forward_only or bias is None:
        grad_bias = None
    zl = torch.empty(nout, dtype=torch.float32, device=dev) if return_z_loss else None
    acc = torch.empty(nout, dtype=torch.float32, device=dev) if return_accuracy else None
    pred = torch.empty(BT, dtype=torch.int64, device=dev) if return_predicted else None
    opt = FlceOptions(int(forward_only), bias.data_ptr() if bias is not None else None,
                      grad_bias.data_ptr() if grad_bias is not None else None,
                      float(z_loss_scale), zl.data_ptr() if zl is not None else None,
                      acc.data_ptr() if acc is not None else None,
                      pred.data_ptr() if pred is not None else None)
    if grad_output is not None:
        grad_output = grad_output.to(device=dev, dtype=torch.float32).contiguous()
    need = flce_workspace_bytes_ex(BT, H, V, dt, cs, chunk_mem_const, opt)
    if need == 0:
        raise FlceError(-1, "flce_workspace_bytes_ex")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = FlceStats()
    rc = flce_fwd_bwd_ex(x.data_ptr(), weight.data_ptr(), target.data_ptr(), BT, H, V, dt,
                         ignore_index, red, cs, chunk_mem_const, adt, int(frozen_weight),
                         int(accumulate_dw), grad_output.data_ptr() if grad_output is not None
                         else None, loss.data_ptr(), dX.data_ptr() if dX is not None else None,
                         dW.data_ptr() if dW is not None else None, workspace.data_ptr(),
                         workspace.numel(), stream, st, opt)
    if rc != 0:
        raise FlceError(rc, "flce_fwd_bwd_ex")
    one = (lambda a: a) if red == NONE else (lambda a: None if a is None else a[0])
    row_index = None
    if return_row_index:
        off = flce_workspace_row_index_offset(BT, H, V, dt, cs, chunk_mem_const, opt)
        row_index = workspace[off:off + 4 * st.n_valid].view(torch.int32)
    return FlceResult(loss=one(loss), dX=dX, dW=None if frozen_weight else dW,
                      stats=st.as_dict(), grad_bias=grad_bias, z_loss=one(zl),
                      accuracy=one(acc), predicted=pred, row_index=row_index)


def scale_cast(src, dtype, scale=None, out=None):
    """``scale * src`` converted to ``dtype`` by the library's kernel (scale: device float)."""
    import torch
    if out is None:
        out = torch.empty(src.shape, dtype=dtype, device=src.device)
    if scale is not None:
        scale = scale.to(device=src.device, dtype=torch.float32).contiguous()
    rc = flce_scale_cast(src.data_ptr(), _dtype_code(src.dtype), out.data_ptr(),
                         _dtype_code(dtype), src.numel(),
                         scale.data_ptr() if scale is not None else None,
                         torch.cuda.current_stream(src.device).cuda_stream)
    if rc != 0:
        raise FlceError(rc, "flce_scale_cast")
    return out


from .autograd import FusedLinearCrossEntropy, fused_linear_cross_entropy  # noqa: E402
from .op import fused_linear_cross_entropy_op  # noqa: E402
