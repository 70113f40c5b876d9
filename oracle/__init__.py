"""CPU oracle for fused linear cross-entropy (fp64).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg may use this package; the product path never does.  It shares
no code with the GPU library and never imports it.

Two implementations of the same plain definition:

* ``flce`` / ``dx_rows`` / ``dw_rows`` / ``lse`` -- explicit fp64 loops in C
  (``flce_oracle.c``, OpenMP over independent rows or vocabulary entries);
* ``lse_matmul`` / ``flce_matmul`` -- the same definition written with numpy
  fp64 matrix products as the one library primitive, for shapes where the
  loop version is too slow.  It is pinned to the loop version on small inputs.

Every input is widened exactly to float64 first (bf16, fp16 and fp32 values
are all representable in fp64).  See ``flce_oracle.c`` for the definition and
the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flce_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

REDUCTIONS = {"mean": 0, "sum": 1, "none": 2}
E_TARGET = -3


def build(force: bool = True) -> str:
    """Compile the loop oracle with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC,
                        "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _bind(path: str):
    """Load a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_threads.restype = I
    lib.oracle_compact.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_compact.restype = I
    lib.oracle_lse.argtypes = [P, P, P, I64, I64, I64, I64, P]
    lib.oracle_lse.restype = I
    lib.oracle_flce.argtypes = [P, P, P, I64, I64, I64, I64, I, P, I, I, P, P, P, P, P]
    lib.oracle_flce.restype = I
    lib.oracle_dx_rows.argtypes = [P, P, P, I64, I64, I64, I, P, I64, P, I64, P, P, P]
    lib.oracle_dx_rows.restype = I
    lib.oracle_dw_rows.argtypes = [P, P, P, I64, I64, I64, I, P, I64, P, I64, P, P]
    lib.oracle_dw_rows.restype = I
    D = ctypes.c_double
    lib.oracle_flce_ex.argtypes = [P, P, P, P, I64, I64, I64, I64, I, P, D, I, P, P, P, P, P, P,
                                   P]
    lib.oracle_flce_ex.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _lib = _bind(LIB_PATH)
    return _lib


class OracleTargetError(ValueError):
    """A labelled target lies outside [0, V)."""


def widen(a) -> np.ndarray:
    """Exact widening of a torch tensor or numpy array to contiguous float64."""
    if hasattr(a, "detach"):  # torch tensor: bf16/fp16 -> fp32 is exact
        a = a.detach().cpu().float().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int64)


def _p(a):
    return None if a is None else a.ctypes.data


def threads() -> int:
    return _load().oracle_threads()


def compact(targets, V: int, ignore_index: int = -100):
    """Ascending list of labelled rows (int64) and its length."""
    t = _i64(targets)
    idx = np.zeros(max(t.size, 1), dtype=np.int64)
    n = np.zeros(1, dtype=np.int64)
    rc = _load().oracle_compact(_p(t), t.size, V, ignore_index, _p(idx), _p(n))
    if rc == E_TARGET:
        raise OracleTargetError("labelled target outside [0, V)")
    return idx[: int(n[0])].copy(), int(n[0])


def _grad(grad_output, reduction: str, BT: int):
    if grad_output is None:
        return None
    g = widen(grad_output).reshape(-1)
    need = BT if reduction == "none" else 1
    if g.size != need:
        raise ValueError(f"grad_output must have {need} element(s), got {g.size}")
    return g


def flce(X, W, targets, *, ignore_index: int = -100, reduction: str = "mean",
         grad_output=None, frozen: bool = False, dW_init=None):
    """Full oracle: loss, dX, dW (None when frozen), lse, n_valid.

    ``dW_init`` given -> dW is added to it (accumulation), else overwritten.
    """
    Xd, Wd, t = widen(X), widen(W), _i64(targets)
    BT, H = Xd.shape
    V = Wd.shape[0]
    g = _grad(grad_output, reduction, BT)
    loss = np.zeros(BT if reduction == "none" else 1, dtype=np.float64)
    dX = np.zeros((BT, H), dtype=np.float64)
    dW = None
    if not frozen:
        dW = np.zeros((V, H), dtype=np.float64) if dW_init is None else widen(dW_init).copy()
    lse = np.zeros(BT, dtype=np.float64)
    n = np.zeros(1, dtype=np.int64)
    rc = _load().oracle_flce(_p(Xd), _p(Wd), _p(t), BT, H, V, ignore_index,
                             REDUCTIONS[reduction], _p(g), int(frozen), int(dW_init is not None),
                             _p(loss), _p(dX), _p(dW), _p(lse), _p(n))
    if rc == E_TARGET:
        raise OracleTargetError("labelled target outside [0, V)")
    if rc != 0:
        raise RuntimeError(f"oracle_flce failed with {rc}")
    return dict(loss=loss if reduction == "none" else float(loss[0]), dX=dX, dW=dW, lse=lse,
                n_valid=int(n[0]))


def flce_ex(X, W, targets, *, bias=None, z_loss_scale: float = 0.0, ignore_index: int = -100,
            reduction: str = "mean", grad_output=None, dW_init=None, db_init=None,
            grads: bool = True):
    """The method with bias, z-loss and per-token outputs (small cases only).

    Returns loss, z_loss, accuracy (scalars for mean/sum, [BT] for none),
    predicted [BT] (int64, -1 at ignored rows) and, with ``grads``, dX, dW and
    grad_bias (when a bias is given).  ``dW_init`` / ``db_init`` turn the
    weight / bias gradients into accumulations onto those values.
    """
    Xd, Wd, t = widen(X), widen(W), _i64(targets)
    BT, H = Xd.shape
    V = Wd.shape[0]
    bd = None if bias is None else widen(bias).reshape(-1)
    g = _grad(grad_output, reduction, BT)
    nout = BT if reduction == "none" else 1
    loss = np.zeros(nout)
    zl = np.zeros(nout)
    acc = np.zeros(nout)
    pred = np.zeros(max(BT, 1), dtype=np.int64)
    accumulate = dW_init is not None or db_init is not None
    dX = np.zeros((BT, H)) if grads else None
    dW = None
    db = None
    if grads:
        dW = np.zeros((V, H)) if dW_init is None else widen(dW_init).copy()
        if bd is not None:
            db = np.zeros(V) if db_init is None else widen(db_init).reshape(-1).copy()
    rc = _load().oracle_flce_ex(_p(Xd), _p(Wd), _p(bd), _p(t), BT, H, V, ignore_index,
                                REDUCTIONS[reduction], _p(g), float(z_loss_scale),
                                int(accumulate), _p(loss), _p(dX), _p(dW), _p(db), _p(zl),
                                _p(acc), _p(pred))
    if rc == E_TARGET:
        raise OracleTargetError("labelled target outside [0, V)")
    if rc != 0:
        raise RuntimeError(f"oracle_flce_ex failed with {rc}")
    red = (lambda a: a) if reduction == "none" else (lambda a: float(a[0]))
    return dict(loss=red(loss), z_loss=red(zl), accuracy=red(acc), predicted=pred[:BT],
                dX=dX, dW=dW, grad_bias=db)


def lse(X, W, targets, *, ignore_index: int = -100) -> np.ndarray:
    """Loop oracle: lse of every row (NaN for ignored rows)."""
    Xd, Wd, t = widen(X), widen(W), _i64(targets)
    out = np.zeros(Xd.shape[0], dtype=np.float64)
    rc = _load().oracle_lse(_p(Xd), _p(Wd), _p(t), Xd.shape[0], Xd.shape[1], Wd.shape[0],
                            ignore_index, _p(out))
    if rc != 0:
        raise RuntimeError(f"oracle_lse failed with {rc}")
    return out


def dx_rows(X, W, targets, rows, *, n_valid: int, ignore_index: int = -100,
            reduction: str = "mean", grad_output=None):
    """Loop oracle on selected rows: (dX rows [R,H], loss rows [R], lse rows [R])."""
    Xd, Wd, t = widen(X), widen(W), _i64(targets)
    r = _i64(rows)
    H, V = Xd.shape[1], Wd.shape[0]
    g = _grad(grad_output, reduction, Xd.shape[0])
    dx = np.zeros((r.size, H), dtype=np.float64)
    lr = np.zeros(r.size, dtype=np.float64)
    ls = np.zeros(r.size, dtype=np.float64)
    rc = _load().oracle_dx_rows(_p(Xd), _p(Wd), _p(t), H, V, ignore_index,
                                REDUCTIONS[reduction], _p(g), n_valid, _p(r), r.size, _p(dx),
                                _p(lr), _p(ls))
    if rc != 0:
        raise RuntimeError(f"oracle_dx_rows failed with {rc}")
    return dx, lr, ls


def dw_rows(X, W, targets, vrows, lse_all, *, n_valid: int, ignore_index: int = -100,
            reduction: str = "mean", grad_output=None):
    """Loop oracle on selected vocabulary rows, given lse of every row: dW rows [R,H]."""
    Xd, Wd, t = widen(X), widen(W), _i64(targets)
    v = _i64(vrows)
    l = np.ascontiguousarray(lse_all, dtype=np.float64)
    BT, H = Xd.shape
    g = _grad(grad_output, reduction, BT)
    dw = np.zeros((v.size, H), dtype=np.float64)
    rc = _load().oracle_dw_rows(_p(Xd), _p(Wd), _p(t), BT, H, ignore_index,
                                REDUCTIONS[reduction], _p(g), n_valid, _p(v), v.size, _p(l),
                                _p(dw))
    if rc != 0:
        raise RuntimeError(f"oracle_dw_rows failed with {rc}")
    return dw


# ---------------------------------------------------------------------------
# Same definition with numpy fp64 matrix products as the library primitive.
# ---------------------------------------------------------------------------

def _logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def lse_matmul(Xd: np.ndarray, Wd: np.ndarray, targets, *, ignore_index: int = -100,
               rows_per_block: int = 512) -> np.ndarray:
    """lse of every labelled row via Z = X_rows @ W^T (fp64); NaN for ignored rows.

    Rows are independent, so they are taken a block at a time only to bound
    memory; within a row nothing is reordered beyond the matmul itself.
    """
    t = _i64(targets)
    out = np.full(Xd.shape[0], np.nan, dtype=np.float64)
    lab = np.nonzero(t != ignore_index)[0]
    WdT = Wd.T
    for s in range(0, lab.size, rows_per_block):
        r = lab[s:s + rows_per_block]
        out[r] = _logsumexp_rows(Xd[r] @ WdT)
    return out


def flce_matmul(X, W, targets, *, ignore_index: int = -100, reduction: str = "mean",
                grad_output=None, frozen: bool = False):
    """Whole-batch definition with matrix products (small shapes only: builds [N,V])."""
    Xd, Wd, t = widen(X), widen(W), _i64(targets)
    BT, H = Xd.shape
    V = Wd.shape[0]
    g = _grad(grad_output, reduction, BT)
    idx, N = compact(t, V, ignore_index)
    Z = Xd[idx] @ Wd.T
    lse_l = _logsumexp_rows(Z) if N else np.zeros(0)
    rows = np.arange(N)
    lrow = lse_l - Z[rows, t[idx]]
    if reduction == "none":
        s = g[idx] if g is not None else np.ones(N)
    else:
        gs = g[0] if g is not None else 1.0
        s = np.full(N, gs / N if (reduction == "mean" and N) else gs)
    G = np.exp(Z - lse_l[:, None])
    G[rows, t[idx]] -= 1.0
    G *= s[:, None]
    dX = np.zeros((BT, H))
    dX[idx] = G @ Wd
    dW = None if frozen else G.T @ Xd[idx]
    if reduction == "none":
        loss = np.zeros(BT)
        loss[idx] = lrow
    else:
        tot = lrow.sum()
        loss = (tot / N if N else 0.0) if reduction == "mean" else tot
    lse_full = np.full(BT, np.nan)
    lse_full[idx] = lse_l
    return dict(loss=loss, dX=dX, dW=dW, lse=lse_full, n_valid=N)


def _row_scales(t, rows, n_valid: int, reduction: str, g):
    """s_i for the given labelled rows: g/N (mean), g (sum), g_i (none)."""
    if reduction == "none":
        return np.ones(rows.size) if g is None else g[rows]
    gs = 1.0 if g is None else float(g[0])
    return np.full(rows.size, gs / n_valid if reduction == "mean" else gs)


def dx_rows_matmul(Xd: np.ndarray, Wd: np.ndarray, targets, rows, *, n_valid: int,
                   ignore_index: int = -100, reduction: str = "mean", grad_output=None,
                   rows_per_block: int = 64):
    """``dx_rows`` with numpy fp64 matrix products: (dX rows [R,H], loss [R], lse [R]).

    Per selected labelled row i: z = X_i W^T, lse, loss = lse - z_t, and
    dX_i = s_i (softmax(z) - onehot(t_i)) W.  Ignored rows give +0.0, loss 0
    and NaN lse.  Blocks of rows only bound memory.
    """
    t = _i64(targets)
    r = _i64(rows)
    g = _grad(grad_output, reduction, Xd.shape[0])
    H = Xd.shape[1]
    dx = np.zeros((r.size, H))
    lr = np.zeros(r.size)
    ls = np.full(r.size, np.nan)
    lab = np.nonzero(t[r] != ignore_index)[0]
    for s0 in range(0, lab.size, rows_per_block):
        sel = lab[s0:s0 + rows_per_block]
        ri = r[sel]
        Z = Xd[ri] @ Wd.T
        l = _logsumexp_rows(Z)
        k = np.arange(sel.size)
        lr[sel] = l - Z[k, t[ri]]
        ls[sel] = l
        G = np.exp(Z - l[:, None])
        G[k, t[ri]] -= 1.0
        G *= _row_scales(t, ri, n_valid, reduction, g)[:, None]
        dx[sel] = G @ Wd
    return dx, lr, ls


def dw_rows_matmul(Xd: np.ndarray, Wd: np.ndarray, targets, vrows, lse_all, *, n_valid: int,
                   ignore_index: int = -100, reduction: str = "mean", grad_output=None,
                   rows_per_block: int = 2048):
    """``dw_rows`` with numpy fp64 matrix products: dW rows [R,H] for vocabulary rows vrows.

    dW_v = sum over labelled i of s_i (exp(z_iv - lse_i) - [t_i == v]) X_i,
    with z_iv = X_i . W_v and lse the given per-row log-sum-exp.  Only labelled
    rows enter (an ignored row is never read).  Row blocks only bound memory;
    each block's product is added in ascending row order.
    """
    t = _i64(targets)
    v = _i64(vrows)
    g = _grad(grad_output, reduction, Xd.shape[0])
    lse_all = np.asarray(lse_all, dtype=np.float64)
    lab = np.nonzero(t != ignore_index)[0]
    out = np.zeros((v.size, Xd.shape[1]))
    Wv = Wd[v]
    for s0 in range(0, lab.size, rows_per_block):
        ri = lab[s0:s0 + rows_per_block]
        Xi = Xd[ri]
        G = np.exp(Xi @ Wv.T - lse_all[ri][:, None])
        G -= (t[ri][:, None] == v[None, :])
        G *= _row_scales(t, ri, n_valid, reduction, g)[:, None]
        out += G.T @ Xi
    return out


def target_logits(Xd: np.ndarray, Wd: np.ndarray, targets, *, ignore_index: int = -100):
    """z[i, t_i] = X_i . W_{t_i} for labelled rows (fp64; 0 for ignored rows)."""
    t = _i64(targets)
    lab = t != ignore_index
    z = np.zeros(Xd.shape[0], dtype=np.float64)
    rows = np.nonzero(lab)[0]
    for s in range(0, rows.size, 4096):
        r = rows[s:s + 4096]
        z[r] = np.einsum("ij,ij->i", Xd[r], Wd[t[r]])
    return z


def loss_from_lse(lse: np.ndarray, zt: np.ndarray, targets, *, ignore_index: int = -100,
                  reduction: str = "mean"):
    """Cross-entropy from per-row lse and target logit: mean/sum scalar, or [BT] for none."""
    t = _i64(targets)
    lab = t != ignore_index
    rows = np.where(lab, lse - zt, 0.0)
    if reduction == "none":
        return rows
    tot = float(np.sum(rows[lab]))
    n = int(lab.sum())
    return (tot / n if n else 0.0) if reduction == "mean" else tot
