"""Seeded random configurations of the optional parts (flce_fwd_bwd_ex) against
the oracle's flce_ex.

Each case draws the operand dtype, the shape, the chunk size, the reduction,
an ignored share and ignore_index, and then which options are on: a bias
(with its gradient), a z-loss coefficient, the per-token outputs (z-loss,
accuracy, predicted token), a loss-only call, and accumulation of the weight
and bias gradients onto random buffers.  Checks as in the fixed cases: loss
and z-loss to the loss tolerance, dX / dW / grad_bias to the gradient
tolerance, exact zeros (and -1 predictions) at ignored rows, the predicted
token equal to the oracle's wherever the top two logits are apart by more
than fp32 accumulation can move, and the accuracy consistent with it.  In
about half the cases the ignored rows of X hold NaN on the GPU (the oracle
gets the clean rows): nothing of them may reach any output (PR #1554, Tests:
ignored rows never enter the projection, with bias on and off).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2), "f16": (2e-3, 2e-2)}
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
N_CASES = 80


def draw(i):
    """The configuration of case i (a pure function of i)."""
    r = np.random.Generator(np.random.PCG64(31337 + i))
    pick = lambda xs: xs[int(r.integers(len(xs)))]
    dtype = pick(["f32", "bf16", "bf16", "f16"])
    BT = int(pick([1, int(r.integers(2, 100)), int(r.integers(100, 420))]))
    H = 8 * int(r.integers(1, 33))
    V = int(pick([2, int(r.integers(3, 100)), int(r.integers(100, 700)),
                  int(r.integers(700, 1300))]))
    return dict(dtype=dtype, BT=BT, H=H, V=V,
                chunk=pick([None, 1, 16, 64, 100, 256, 512]),
                reduction=pick(["mean", "sum", "none"]),
                ignore=pick(["none", "scattered", "scattered", "prompt_first"]),
                frac=float(pick([0.1, 0.4, 0.8])),
                ignore_index=-100 if r.random() < 0.7 else int(r.integers(0, V)),
                bias=bool(r.random() < 0.6),
                lam=float(pick([0.0, 1e-4, 1e-3])),
                forward_only=bool(r.random() < 0.25),
                want_z=bool(r.random() < 0.6), want_acc=bool(r.random() < 0.6),
                want_pred=bool(r.random() < 0.6),
                accumulate=bool(r.random() < 0.2),
                seed=8000 + 13 * i,
                poison=bool(r.random() < 0.5))


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def _check_predicted(pred, ref_pred, z, lab, margin=1e-4):
    assert np.all(pred[~lab] == -1)
    for i in np.nonzero(lab)[0]:
        zi = z[i]
        mx = zi.max()
        scale = max(np.abs(zi).max(), 1e-30)
        top2 = np.sort(zi)[-2] if zi.size > 1 else -np.inf
        if mx - top2 > margin * scale:
            assert pred[i] == ref_pred[i], (i, pred[i], ref_pred[i])
        else:
            assert 0 <= pred[i] < zi.size and zi[pred[i]] >= mx - margin * scale, i


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_options(pkg, i):
    c = draw(i)
    dt, BT, H, V, ii = c["dtype"], c["BT"], c["H"], c["V"], c["ignore_index"]
    print(f"case {i}: {c}", flush=True)
    X = si.make_x(BT, H, dt, c["seed"])
    W = si.make_w(V, H, dt, c["seed"], scale=0.5 if dt == "f32" else 0.1)
    t = si.make_targets(BT, V, c["seed"], ignore=c["ignore"], frac=c["frac"], ignore_index=ii)
    lab = (t != ii).numpy()
    b = (si.make_x(1, V, "f32", c["seed"] + 7).reshape(-1) * 0.5).to(TD[dt]) if c["bias"] else None
    red = c["reduction"]
    g = si.make_grad_output(t, red, c["seed"], scalar=0.75, ignore_index=ii)
    grads = not c["forward_only"]
    acc_dt = torch.float32
    rng = np.random.Generator(np.random.PCG64(c["seed"] + 9))
    dW0 = db0 = None
    if grads and c["accumulate"]:
        dW0 = torch.from_numpy(rng.standard_normal((V, H)).astype(np.float32) * 0.01)
        if b is not None:
            db0 = torch.from_numpy(rng.standard_normal(V).astype(np.float32) * 0.01)

    dev = torch.device("cuda:0")
    Xg = X.clone()
    if c["poison"] and (~lab).any():
        Xg[torch.from_numpy(~lab)] = float("nan")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        Xg.to(dev), W.to(dev), t.to(dev), bias=None if b is None else b.to(dev), ignore_index=ii,
        reduction=red, chunk_size=c["chunk"], accum_dtype=acc_dt, grad_output=g.to(dev),
        forward_only=c["forward_only"], z_loss_scale=c["lam"], return_z_loss=c["want_z"],
        return_accuracy=c["want_acc"], return_predicted=c["want_pred"],
        dW=None if dW0 is None else dW0.clone().to(dev),
        grad_bias=None if db0 is None else db0.clone().to(dev),
        accumulate_dw=dW0 is not None)
    torch.cuda.synchronize()
    assert r.stats["n_valid"] == int(lab.sum())

    ref = oracle.flce_ex(X, W, t, bias=b, z_loss_scale=c["lam"], ignore_index=ii, reduction=red,
                         grad_output=torch.nan_to_num(g).numpy(), dW_init=dW0, db_init=db0,
                         grads=grads)
    tl, tg = TOL[dt]

    def close_loss(got, want):
        if red == "none":
            got = got.cpu().numpy()
            assert np.all(got[~lab] == 0.0) and not np.signbit(got[~lab]).any()
            assert _rel(got[lab], want[lab]) <= tl
        else:
            assert abs(float(got) - want) <= tl * max(abs(want), 1e-30), (float(got), want)

    if lab.any():
        close_loss(r.loss, ref["loss"])
        if c["want_z"]:
            close_loss(r.z_loss, ref["z_loss"])
    else:
        assert np.all(r.loss.cpu().numpy() == 0.0)
    if grads:
        dx = r.dX.float().cpu().numpy()
        assert np.all(dx[~lab] == 0.0) and not np.signbit(dx[~lab]).any()
        assert _rel(dx, ref["dX"]) <= tg
        assert _rel(r.dW.double().cpu().numpy(), ref["dW"]) <= tg
        if b is not None:
            assert _rel(r.grad_bias.double().cpu().numpy(), ref["grad_bias"]) <= tg

    if c["want_pred"] or c["want_acc"]:
        Xd, Wd = oracle.widen(X), oracle.widen(W)
        z = Xd @ Wd.T + (0.0 if b is None else oracle.widen(b)[None, :])
    if c["want_pred"]:
        pred = r.predicted.cpu().numpy()
        _check_predicted(pred, ref["predicted"], z, lab)
        if c["want_acc"]:
            acc_tok = np.where(lab, (pred == t.numpy()).astype(np.float64), 0.0)
            if red == "none":
                np.testing.assert_array_equal(r.accuracy.cpu().numpy(), acc_tok)
            else:
                n = max(lab.sum(), 1) if red == "mean" else 1.0
                assert float(r.accuracy) == pytest.approx(acc_tok.sum() / n, rel=1e-6, abs=1e-7)
    elif c["want_acc"]:
        # accuracy alone: compare with the oracle's wherever the argmax is unambiguous
        if red == "none":
            got = r.accuracy.cpu().numpy()
            assert np.all(got[~lab] == 0.0)
            zs = np.sort(z, axis=1)
            clear = lab & ((zs[:, -1] - zs[:, -2]) > 1e-4 * np.abs(z).max(axis=1))
            np.testing.assert_array_equal(got[clear], ref["accuracy"][clear])
