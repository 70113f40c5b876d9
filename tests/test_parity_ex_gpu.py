"""GPU parity of the optional parts (flce_fwd_bwd_ex) against the oracle's flce_ex.

Covers bias and grad_bias, the z-loss coefficient, the per-token outputs
(z-loss, accuracy, predicted token) and the loss-only call, at sizes that span
several GEMM tiles, several chunks and ragged tails.

Tolerances as for the other parity tests: fp32 loss 1e-5, gradients 1e-4;
bf16 loss 2e-3, gradients 2e-2 (relative Frobenius).  The predicted token is
an argmax decided in fp32 by the kernel: it must equal the oracle's wherever
the oracle's top-two logit gap exceeds what fp32 accumulation can move
(1e-4 relative to the row's largest |logit| here), and elsewhere it must be a
column whose exact logit is within that margin of the maximum.  Exact ties
(duplicate vocabulary rows, inside one 64-column block and across blocks)
must resolve to the lower index.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2)}
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


def _case(BT, H, V, dtype, seed, frac=0.2, ties=False):
    X = si.make_x(BT, H, dtype, seed)
    W = si.make_w(V, H, dtype, seed, scale=0.5 if dtype == "f32" else 0.1)
    t = si.make_targets(BT, V, seed, ignore="scattered", frac=frac)
    b = (si.make_x(1, V, "f32", seed + 7).reshape(-1) * 0.5).to(TD[dtype])
    if ties:
        W = W.clone()
        b = b.clone()
        W[5] = W[2]      # tie inside the first 64-column block
        b[5] = b[2]
        W[200] = W[70]   # tie across blocks
        b[200] = b[70]
    return X, W, t, b


def _check_predicted(pred, ref_pred, Xd, Wd, bd, t, margin=1e-4):
    lab = t != -100
    assert np.all(pred[~lab] == -1)
    z = Xd @ Wd.T + bd[None, :]
    for i in np.nonzero(lab)[0]:
        zi = z[i]
        mx = zi.max()
        scale = max(np.abs(zi).max(), 1e-30)
        top2 = np.sort(zi)[-2] if zi.size > 1 else -np.inf
        if mx - top2 > margin * scale:
            assert pred[i] == ref_pred[i], (i, pred[i], ref_pred[i])
        else:
            assert 0 <= pred[i] < zi.size and zi[pred[i]] >= mx - margin * scale, i


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("chunk", [64, 0])
def test_bias_zloss_and_outputs(pkg, dtype, reduction, chunk):
    BT, H, V = 300, 96, 700
    X, W, t, b = _case(BT, H, V, dtype, seed=17)
    lam = 1e-3
    g = si.make_grad_output(t, "none", 17, scalar=1.0) if reduction == "none" else None
    dev = torch.device("cuda:0")
    accum = torch.float32
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction=reduction,
        chunk_size=chunk or None, accum_dtype=accum, z_loss_scale=lam,
        grad_output=None if g is None else g.to(dev), return_z_loss=True,
        return_accuracy=True, return_predicted=True)
    torch.cuda.synchronize()
    ref = oracle.flce_ex(X, W, t, bias=b, z_loss_scale=lam, reduction=reduction,
                         grad_output=None if g is None else g.numpy())
    tl, tg = TOL[dtype]
    lab = (t != -100).numpy()
    if reduction == "none":
        loss = r.loss.cpu().numpy()
        assert np.all(loss[~lab] == 0.0)
        assert _rel(loss[lab], ref["loss"][lab]) <= tl
        zl = r.z_loss.cpu().numpy()
        assert np.all(zl[~lab] == 0.0)
        assert _rel(zl[lab], ref["z_loss"][lab]) <= tl
    else:
        assert abs(float(r.loss) - ref["loss"]) <= tl * abs(ref["loss"])
        assert abs(float(r.z_loss) - ref["z_loss"]) <= tl * abs(ref["z_loss"])
    assert _rel(r.dX.double().cpu(), ref["dX"]) <= tg
    assert np.all(r.dX.float().cpu().numpy()[~lab] == 0.0)
    assert _rel(r.dW.double().cpu(), ref["dW"]) <= tg
    assert _rel(r.grad_bias.double().cpu(), ref["grad_bias"]) <= tg

    pred = r.predicted.cpu().numpy()
    Xd, Wd, bd = oracle.widen(X), oracle.widen(W), oracle.widen(b)
    _check_predicted(pred, ref["predicted"], Xd, Wd, bd, t.numpy())
    acc_tok = np.where(lab, (pred == t.numpy()).astype(np.float64), 0.0)
    if reduction == "none":
        np.testing.assert_array_equal(r.accuracy.cpu().numpy(), acc_tok)
    else:
        n = lab.sum() if reduction == "mean" else 1.0
        assert float(r.accuracy) == pytest.approx(acc_tok.sum() / n, rel=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_poisoned_ignored_rows_with_every_option(pkg, dtype, reduction):
    """NaN and Inf in ignored X rows (and NaN in the upstream gradient there),
    with the bias, a z-loss coefficient and every per-token output on: every
    output bit-identical to the clean run, and within tolerance of the oracle
    (PR #1554, Tests: ignored rows never enter the projection, with bias on
    and off)."""
    BT, H, V = 300, 96, 700
    X, W, t, b = _case(BT, H, V, dtype, seed=29, frac=0.3)
    lab = (t != -100).numpy()
    ign = np.nonzero(~lab)[0]
    Xp = X.clone()
    Xp[torch.from_numpy(ign[0::2])] = float("nan")
    Xp[torch.from_numpy(ign[1::2])] = float("inf")
    lam = 1e-3
    g = si.make_grad_output(t, "none", 29, scalar=1.0) if reduction == "none" else None
    dev = torch.device("cuda:0")

    def run(x):
        r = pkg.fused_linear_cross_entropy_fwd_bwd(
            x.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction=reduction,
            chunk_size=64, accum_dtype=torch.float32, z_loss_scale=lam,
            grad_output=None if g is None else g.to(dev), return_z_loss=True,
            return_accuracy=True, return_predicted=True)
        torch.cuda.synchronize()
        return {k: getattr(r, k).cpu() for k in
                ("loss", "z_loss", "accuracy", "predicted", "dX", "dW", "grad_bias")}

    clean, pois = run(X), run(Xp)
    for k in clean:
        assert torch.isfinite(pois[k].double()).all(), k
        assert clean[k].reshape(-1).view(torch.uint8).equal(pois[k].reshape(-1).view(torch.uint8)), k
    gref = None if g is None else torch.nan_to_num(g).numpy()
    ref = oracle.flce_ex(X, W, t, bias=b, z_loss_scale=lam, reduction=reduction,
                         grad_output=gref)
    tl, tg = TOL[dtype]
    if reduction == "none":
        assert _rel(pois["loss"].numpy()[lab], ref["loss"][lab]) <= tl
    else:
        assert abs(float(pois["loss"]) - ref["loss"]) <= tl * abs(ref["loss"])
    assert np.all(pois["dX"].float().numpy()[~lab] == 0.0)
    assert _rel(pois["dX"].double(), ref["dX"]) <= tg
    assert _rel(pois["dW"].double(), ref["dW"]) <= tg
    assert _rel(pois["grad_bias"].double(), ref["grad_bias"]) <= tg
    assert np.all(pois["predicted"].numpy()[~lab] == -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ties_resolve_to_lower_index(pkg, dtype):
    BT, H, V = 130, 64, 300
    X, W, t, b = _case(BT, H, V, dtype, seed=23, frac=0.0, ties=True)
    # make the duplicated columns the row maxima: large equal bias
    b = b.clone()
    b[2] = b[5] = 40.0
    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction="none", chunk_size=64,
        forward_only=True, return_predicted=True)
    pred = r.predicted.cpu().numpy()
    assert np.all(pred == 2), np.unique(pred)
    b[2] = b[5] = 0.0
    b[70] = b[200] = 40.0
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction="none", chunk_size=64,
        forward_only=True, return_predicted=True)
    assert np.all(r.predicted.cpu().numpy() == 70)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_forward_only_matches_full_call(pkg, reduction):
    BT, H, V = 260, 64, 520
    X, W, t, b = _case(BT, H, V, "bf16", seed=31)
    dev = torch.device("cuda:0")
    args = (X.to(dev), W.to(dev), t.to(dev))
    full = pkg.fused_linear_cross_entropy_fwd_bwd(*args, bias=b.to(dev), reduction=reduction,
                                                  chunk_size=64, return_z_loss=True,
                                                  return_accuracy=True, return_predicted=True)
    fwd = pkg.fused_linear_cross_entropy_fwd_bwd(*args, bias=b.to(dev), reduction=reduction,
                                                 chunk_size=64, forward_only=True,
                                                 return_z_loss=True, return_accuracy=True,
                                                 return_predicted=True)
    torch.cuda.synchronize()
    assert fwd.dX is None and fwd.dW is None and fwd.grad_bias is None
    for name in ("loss", "z_loss", "accuracy", "predicted"):
        assert torch.equal(getattr(fwd, name), getattr(full, name)), name
    ws_full = pkg.flce_workspace_bytes_ex(BT, H, V, pkg.BF16, 64, 1, None)
    ws_fwd = pkg.flce_workspace_bytes_ex(BT, H, V, pkg.BF16, 64, 1, pkg.FlceOptions(1))
    assert ws_fwd < ws_full


def test_plain_call_unchanged_by_zero_options(pkg):
    """A zero options struct gives bit-identical results to flce_fwd_bwd."""
    BT, H, V = 200, 64, 400
    X, W, t, _ = _case(BT, H, V, "bf16", seed=5)
    dev = torch.device("cuda:0")
    args = (X.to(dev), W.to(dev), t.to(dev))
    a = pkg.fused_linear_cross_entropy_fwd_bwd(*args, chunk_size=64, accum_dtype=torch.float32)
    b = pkg.fused_linear_cross_entropy_fwd_bwd(*args, chunk_size=64, accum_dtype=torch.float32,
                                               return_predicted=True, z_loss_scale=0.0)
    torch.cuda.synchronize()
    assert torch.equal(a.loss, b.loss) and torch.equal(a.dX, b.dX) and torch.equal(a.dW, b.dW)


def test_grad_bias_accumulates_and_frozen_weight(pkg):
    BT, H, V = 180, 64, 333
    X, W, t, b = _case(BT, H, V, "f32", seed=9)
    dev = torch.device("cuda:0")
    db0 = torch.full((V,), 0.5, dtype=torch.float32, device=dev)
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction="sum", chunk_size=64,
        frozen_weight=True, grad_bias=db0.clone(), accumulate_dw=True)
    torch.cuda.synchronize()
    ref = oracle.flce_ex(X, W, t, bias=b, reduction="sum", db_init=np.full(V, 0.5))
    assert r.dW is None
    assert _rel(r.grad_bias.double().cpu(), ref["grad_bias"]) <= 1e-4
    assert _rel(r.dX.double().cpu(), ref["dX"]) <= 1e-4


def test_all_rows_ignored_with_options(pkg):
    BT, H, V = 70, 32, 100
    X, W, t, b = _case(BT, H, V, "f32", seed=4, frac=1.0)
    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction="mean", chunk_size=32,
        return_z_loss=True, return_accuracy=True, return_predicted=True)
    torch.cuda.synchronize()
    assert float(r.loss) == 0.0 and float(r.z_loss) == 0.0 and float(r.accuracy) == 0.0
    assert torch.all(r.predicted == -1)
    assert torch.all(r.grad_bias == 0) and torch.all(r.dW == 0) and torch.all(r.dX == 0)


def test_mi355x_policy_is_an_explicit_chunk(pkg):
    """chunk_size="mi355x" runs exactly as the chunk size the policy returns."""
    BT, H, V = 640, 64, 500
    X, W, t, _ = _case(BT, H, V, "bf16", seed=12)
    dev = torch.device("cuda:0")
    args = (X.to(dev), W.to(dev), t.to(dev))
    c = pkg.flce_chunk_size_mi355x(BT, H, V, pkg.BF16, pkg.F32, 0, 0)
    a = pkg.fused_linear_cross_entropy_fwd_bwd(*args, chunk_size="mi355x",
                                               accum_dtype=torch.float32)
    b = pkg.fused_linear_cross_entropy_fwd_bwd(*args, chunk_size=c, accum_dtype=torch.float32)
    torch.cuda.synchronize()
    assert a.stats["chunk_size"] == c
    assert torch.equal(a.loss, b.loss) and torch.equal(a.dX, b.dX) and torch.equal(a.dW, b.dW)


def test_full_size_llama_bias_zloss_outputs(pkg):
    """The optional parts at the Llama-3-8B lm_head shape (bf16, BT 8192,
    H 4096, V 128256, chunk 2048, reduction none, 5 % of rows ignored): the
    loss, z-loss, predicted token and accuracy of sampled rows (three labelled,
    one ignored) against the oracle's forward run on those rows alone; with
    reduction none each of these depends on its own row only.  (The oracle's
    loops take about ten seconds for four rows at this size; the gradients
    with bias and z-loss are compared in full at the smaller sizes above.)"""
    BT, H, V, seed = 8192, 4096, 128256, 1001
    X = si.make_x(BT, H, "bf16", seed)
    W = si.make_w(V, H, "bf16", seed)
    t = si.make_targets(BT, V, seed, ignore="scattered", frac=0.05)
    b = (si.make_x(1, V, "f32", seed + 7).reshape(-1) * 0.5).to(torch.bfloat16)
    lam = 1e-4
    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction="none", chunk_size=2048,
        accum_dtype=torch.float32, z_loss_scale=lam, forward_only=True, return_z_loss=True,
        return_accuracy=True, return_predicted=True)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(11))
    lab_all = (t != -100).numpy()
    rows = np.sort(np.concatenate([rng.choice(np.nonzero(lab_all)[0], 3, replace=False),
                                   np.nonzero(~lab_all)[0][:1]]))
    tr = t[rows]
    ref = oracle.flce_ex(X[rows], W, tr, bias=b, z_loss_scale=lam, reduction="none",
                         grads=False)
    lab = (tr != -100).numpy()
    loss = r.loss.cpu().numpy()[rows]
    zl = r.z_loss.cpu().numpy()[rows]
    assert np.all(loss[~lab] == 0.0) and np.all(zl[~lab] == 0.0)
    assert _rel(loss[lab], ref["loss"][lab]) <= 2e-3
    assert _rel(zl[lab], ref["z_loss"][lab]) <= 2e-3
    pred = r.predicted.cpu().numpy()[rows]
    Xd, Wd, bd = oracle.widen(X[rows]), oracle.widen(W), oracle.widen(b)
    _check_predicted(pred, ref["predicted"], Xd, Wd, bd, tr.numpy())
    acc = r.accuracy.cpu().numpy()[rows]
    np.testing.assert_array_equal(acc, np.where(lab, (pred == tr.numpy()).astype(np.float64), 0.0))


@pytest.mark.parametrize("dtype,shift", [("bf16", 48.0), ("f16", 1000.0), ("f32", 48.0)])
def test_constant_logit_shift_leaves_gradients(pkg, dtype, shift):
    """Adding one constant to every logit (a constant bias) leaves the softmax,
    and so the gradients, unchanged.  At |z| of 48 (bf16) or 1000 (fp16) a
    logit rounded to the operand dtype is off by up to 0.125 / 0.25, which would
    move exp(z - lse) by 13-28 %; the slab keeps z minus its block maximum
    instead, so the gradients still meet the 16-bit tolerance.  The row
    targets are the argmax of each row, so p_target is large and its gradient
    1 - p_target small: the case most sensitive to that rounding."""
    BT, H, V = 96, 64, 500
    X = si.make_x(BT, H, dtype, 51)
    W = si.make_w(V, H, dtype, 51, scale=0.6)
    z = oracle.widen(X) @ oracle.widen(W).T
    t = torch.from_numpy(z.argmax(axis=1).astype(np.int64))
    b = torch.full((V,), shift, dtype=TD[dtype])
    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), bias=b.to(dev), reduction="sum", chunk_size=32,
        accum_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.flce_ex(X, W, t, bias=b, reduction="sum")
    tl, tg = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2), "f16": (2e-3, 2e-2)}[dtype]
    assert abs(float(r.loss) - ref["loss"]) <= tl * abs(ref["loss"])
    assert _rel(r.dX.double().cpu(), ref["dX"]) <= tg
    assert _rel(r.dW.double().cpu(), ref["dW"]) <= tg
    assert _rel(r.grad_bias.double().cpu(), ref["grad_bias"]) <= tg
