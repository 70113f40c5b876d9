"""Pins for the oracle's optional parts (oracle_flce_ex): bias, z-loss and the
per-token outputs.  Each is checked against something other than the oracle:

* torch CPU fp64 autograd of F.linear(x, W, b) + F.cross_entropy (library routine),
  with the z-loss term lam * logsumexp(z)^2 added in torch;
* numpy argmax of torch-computed logits (predicted token, accuracy), including
  exact ties, which must resolve to the lowest index;
* closed forms: W = 0 and b = 0 give lse = log V, z-loss = (log V)^2, and
  predicted token 0 in every row;
* invariants: without a z-loss term the bias gradient sums to zero over the
  vocabulary; with no bias and lam = 0 the extended oracle equals the base one;
* ignored rows: 0 loss, z-loss and accuracy, -1 predicted token (PR #1554,
  Details item 1), and NaN or Inf placed in ignored X rows (and NaN in the
  per-token upstream gradient there) changes no output bit, with the bias on
  and a z-loss coefficient (PR #1554, Tests: ignored rows never enter the
  projection; the ignored-row cases run with bias on and off);
* planted mistakes in the new code must fail these pins.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import synthetic_inputs as si


def _case(BT, H, V, seed, frac=0.25, wscale=0.5):
    X = si.make_x(BT, H, "f32", seed)
    W = si.make_w(V, H, "f32", seed, scale=wscale)
    t = si.make_targets(BT, V, seed, ignore="scattered", frac=frac)
    b = si.make_x(1, V, "f32", seed + 7).reshape(-1) * 0.3
    return X, W, t, b


def _torch_ref(X, W, b, t, reduction, lam=0.0, g=None):
    """fp64 torch: loss (with lam * lse^2 per labelled row), and autograd grads."""
    Xd = torch.tensor(np.asarray(X, dtype=np.float64), requires_grad=True)
    Wd = torch.tensor(np.asarray(W, dtype=np.float64), requires_grad=True)
    bd = None if b is None else torch.tensor(np.asarray(b, dtype=np.float64), requires_grad=True)
    tt = torch.as_tensor(np.asarray(t), dtype=torch.int64)
    z = torch.nn.functional.linear(Xd, Wd, bd)
    ce = torch.nn.functional.cross_entropy(z, tt, ignore_index=-100, reduction="none")
    lab = (tt != -100).double()
    per = ce + lam * torch.logsumexp(z, dim=1) ** 2 * lab
    if reduction == "none":
        loss = per
        gg = torch.as_tensor(np.asarray(g, dtype=np.float64)) if g is not None else torch.ones_like(per)
        (per * gg).sum().backward()
    else:
        loss = per.sum() / (lab.sum() if reduction == "mean" else 1.0)
        loss.backward()
    return (loss.detach().numpy(), Xd.grad.numpy(), Wd.grad.numpy(),
            None if bd is None else bd.grad.numpy(), z.detach().numpy())


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("lam", [0.0, 0.05])
def test_ex_against_torch(oracle_mod, reduction, lam):
    X, W, t, b = _case(BT=37, H=11, V=23, seed=91)
    g = si.make_grad_output(t, "none", 91, scalar=1.0) if reduction == "none" else None
    r = oracle_mod.flce_ex(X, W, t, bias=b, z_loss_scale=lam, reduction=reduction,
                           grad_output=None if g is None else g.numpy())
    loss, dx, dw, db, _ = _torch_ref(X, W, b, t, reduction, lam,
                                     None if g is None else np.where(t.numpy() != -100, g.numpy(), 0.0))
    np.testing.assert_allclose(r["loss"], loss, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dX"], dx, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dW"], dw, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["grad_bias"], db, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_ex_per_token_outputs(oracle_mod, reduction):
    X, W, t, b = _case(BT=53, H=9, V=17, seed=5, frac=0.3)
    # exact ties: vocabulary rows 3 and 11 identical, with equal bias
    W = W.clone()
    W[11] = W[3]
    b = b.clone()
    b[11] = b[3]
    r = oracle_mod.flce_ex(X, W, t, bias=b, reduction=reduction)
    _, _, _, _, z = _torch_ref(X, W, b, t, "sum")
    tn = t.numpy()
    lab = tn != -100
    pred = np.argmax(z, axis=1)  # numpy returns the first maximum
    pred = np.where(lab, pred, -1)
    np.testing.assert_array_equal(r["predicted"], pred)
    assert not np.any(pred == 11), "a tie must resolve to the lower index"
    acc = np.where(lab, (pred == tn).astype(np.float64), 0.0)
    lse = np.where(lab, np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) + z.max(1), 0.0)
    zl = lse ** 2
    if reduction == "none":
        np.testing.assert_array_equal(r["accuracy"], acc)
        np.testing.assert_allclose(r["z_loss"], zl, rtol=1e-13)
        assert np.all(r["z_loss"][~lab] == 0.0) and np.all(r["loss"][~lab] == 0.0)
    else:
        d = lab.sum() if reduction == "mean" else 1.0
        assert r["accuracy"] == pytest.approx(acc.sum() / d, rel=1e-15)
        assert r["z_loss"] == pytest.approx(zl.sum() / d, rel=1e-12)


def test_ex_ties_pick_lowest_index(oracle_mod):
    """Every vocabulary row equal: the predicted token is 0 for every labelled row."""
    X, W, t, b = _case(BT=9, H=5, V=6, seed=3, frac=0.0)
    W = W[:1].repeat(6, 1)
    r = oracle_mod.flce_ex(X, W, t, bias=np.zeros(6), reduction="none")
    np.testing.assert_array_equal(r["predicted"], np.zeros(9, dtype=np.int64))


def test_ex_zero_weight_closed_form(oracle_mod):
    X, W, t, _ = _case(BT=12, H=4, V=10, seed=8, frac=0.25)
    W = W * 0
    r = oracle_mod.flce_ex(X, W, t, bias=np.zeros(10), z_loss_scale=0.1, reduction="none")
    lab = t.numpy() != -100
    L = math.log(10)
    np.testing.assert_allclose(r["z_loss"][lab], L * L, rtol=1e-15)
    np.testing.assert_allclose(r["loss"][lab], L + 0.1 * L * L, rtol=1e-15)
    np.testing.assert_array_equal(r["predicted"], np.where(lab, 0, -1))
    np.testing.assert_array_equal(r["accuracy"], np.where(lab & (t.numpy() == 0), 1.0, 0.0))


def test_ex_bias_grad_sums_to_zero_without_z_loss(oracle_mod):
    X, W, t, b = _case(BT=30, H=6, V=40, seed=12)
    r = oracle_mod.flce_ex(X, W, t, bias=b, reduction="sum")
    assert abs(r["grad_bias"].sum()) <= 1e-12 * np.abs(r["grad_bias"]).sum()


def test_ex_reduces_to_base_oracle(oracle_mod):
    X, W, t, _ = _case(BT=25, H=7, V=13, seed=44)
    for red in ("mean", "sum", "none"):
        a = oracle_mod.flce_ex(X, W, t, reduction=red)
        f = oracle_mod.flce(X, W, t, reduction=red)
        np.testing.assert_allclose(a["loss"], f["loss"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(a["dX"], f["dX"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(a["dW"], f["dW"], rtol=1e-12, atol=1e-15)


def test_ex_accumulates(oracle_mod):
    X, W, t, b = _case(BT=20, H=5, V=9, seed=61)
    base = oracle_mod.flce_ex(X, W, t, bias=b, reduction="sum")
    dw0 = np.full_like(base["dW"], 0.25)
    db0 = np.full_like(base["grad_bias"], -0.5)
    acc = oracle_mod.flce_ex(X, W, t, bias=b, reduction="sum", dW_init=dw0, db_init=db0)
    np.testing.assert_allclose(acc["dW"], dw0 + base["dW"], rtol=1e-14)
    np.testing.assert_allclose(acc["grad_bias"], db0 + base["grad_bias"], rtol=1e-14)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_ex_nan_in_ignored_rows_changes_nothing(oracle_mod, reduction, with_bias):
    """Poisoned ignored rows: every output bit-identical to the clean run, all finite."""
    X, W, t, b = _case(BT=12, H=4, V=7, seed=17, frac=0.34)
    tn = t.numpy()
    ign = np.nonzero(tn == -100)[0]
    assert ign.size >= 4
    Xp = X.clone()
    Xp[ign[0::2]] = float("nan")
    Xp[ign[1::2]] = float("inf")
    bias = b if with_bias else None
    g = None
    gp = None
    if reduction == "none":
        g = si.make_grad_output(t, "none", 17, scalar=1.0).numpy()
        g = np.where(tn != -100, g, 0.5)
        gp = np.where(tn != -100, g, np.nan)
    kw = dict(bias=bias, z_loss_scale=0.05, reduction=reduction)
    clean = oracle_mod.flce_ex(X, W, t, grad_output=g, **kw)
    pois = oracle_mod.flce_ex(Xp, W, t, grad_output=gp, **kw)
    for key in ("loss", "z_loss", "accuracy", "predicted", "dX", "dW", "grad_bias"):
        a, c = clean[key], pois[key]
        if a is None:
            assert c is None and (key != "grad_bias" or not with_bias)
            continue
        a, c = np.asarray(a), np.asarray(c)
        assert np.all(np.isfinite(c)), f"{key} not finite after poisoning ignored rows"
        assert a.tobytes() == c.tobytes(), f"{key} changed by poisoned ignored rows"
    assert np.all(pois["dX"][ign] == 0.0) and not np.any(np.signbit(pois["dX"][ign]))


# ------------------------------------------------------------ planted mistakes
MUTANTS_EX = [
    ("bias left out of the logits", "z[v] += bias[v];", "z[v] += 0.0 * bias[v];"),
    ("z-loss gradient sign flipped", "(1.0 + 2.0 * lam * l)", "(1.0 - 2.0 * lam * l)"),
    ("z-loss missing from the loss", "lrow[i] = l - z[t[i]] + lam * l * l;",
     "lrow[i] = l - z[t[i]];"),
    ("ties resolve to the last index", "if (z[v] > z[am]) am = v;", "if (z[v] >= z[am]) am = v;"),
    ("grad_bias sums the wrong column", "for (int64_t n = 0; n < N; ++n) a += G[idx[n] * V + v];",
     "for (int64_t n = 0; n < N; ++n) a += G[idx[n] * V + (v + 1) % V];"),
    ("grad_weight sums over every row, ignored ones included",
     "for (int64_t n = 0; n < N; ++n) a += G[idx[n] * V + v] * X[idx[n] * H + k];",
     "for (int64_t i = 0; i < BT; ++i) a += G[i * V + v] * X[i * H + k];"),
    ("accuracy reduced by the wrong count", "if (acc) acc[0] = d > 0.0 ? sa / d : 0.0;",
     "if (acc) acc[0] = d > 0.0 ? sa / (d + 1.0) : 0.0;"),
]


def _ex_pins_pass(oracle_mod) -> bool:
    try:
        for red in ("mean", "sum", "none"):
            for lam in (0.0, 0.05):
                test_ex_against_torch(oracle_mod, red, lam)
            test_ex_per_token_outputs(oracle_mod, red)
        test_ex_ties_pick_lowest_index(oracle_mod)
        for red in ("mean", "sum", "none"):
            test_ex_nan_in_ignored_rows_changes_nothing(oracle_mod, red, True)
    except AssertionError:
        return False
    return True


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", MUTANTS_EX, ids=[m[0] for m in MUTANTS_EX])
def test_ex_planted_mistake_is_caught(oracle_mod, tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "flce_oracle.c")).read()
    assert old in src, f"mutation site for {name!r} not found"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new, 1))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(mut), "-lm"],
                   check=True)
    saved = oracle_mod._lib
    try:
        oracle_mod._lib = oracle_mod._bind(str(so))
        assert not _ex_pins_pass(oracle_mod), f"planted mistake not caught: {name}"
    finally:
        oracle_mod._lib = saved
    assert _ex_pins_pass(oracle_mod)
