"""Pins for the fp64 CPU oracle: each checks it against something other than itself.

* hand-derived tiny cases (tests/golden/hand_cases.json);
* a textbook library routine: torch CPU fp64 cross_entropy + autograd;
* closed forms (W = 0, X = 0, two classes = softplus);
* central finite differences of the loss;
* invariants (softmax - onehot rows sum to zero, common shift of W rows,
  block additivity = chunk invariance, reduction relations);
* ignored rows: zero outputs, and NaN placed there never reaching anything;
* planted mistakes in the oracle's C source must fail these pins.
"""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(BT, H, V, seed, dtype="f32", frac=0.0, ignore="scattered", wscale=0.5):
    X = si.make_x(BT, H, dtype, seed)
    W = si.make_w(V, H, dtype, seed, scale=wscale)
    t = si.make_targets(BT, V, seed, ignore=ignore, frac=frac)
    return X, W, t


def _torch_ref(X, W, t, reduction, g=None, ignore_index=-100):
    """Library routine in fp64: F.cross_entropy on X W^T, gradients by autograd."""
    Xd = torch.tensor(np.asarray(X, dtype=np.float64), requires_grad=True)
    Wd = torch.tensor(np.asarray(W, dtype=np.float64), requires_grad=True)
    tt = torch.as_tensor(np.asarray(t), dtype=torch.int64)
    loss = torch.nn.functional.cross_entropy(Xd @ Wd.T, tt, ignore_index=ignore_index,
                                             reduction=reduction)
    if reduction == "none":
        gg = torch.tensor(np.where(np.asarray(t) == ignore_index, 0.0,
                                   np.nan_to_num(np.asarray(g, dtype=np.float64))))
        obj = (loss * gg).sum()
    else:
        obj = loss * (float(g[0]) if g is not None else 1.0)
    obj.backward()
    return loss.detach().numpy(), Xd.grad.numpy(), Wd.grad.numpy()


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ---------------------------------------------------------------- hand cases
def test_hand_cases(oracle_mod):
    cases = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))["cases"]
    for c in cases:
        g = None if c["grad_output"] is None else np.array(c["grad_output"], dtype=np.float32)
        out = oracle_mod.flce(np.array(c["X"]), np.array(c["W"]), np.array(c["targets"]),
                              reduction=c["reduction"], grad_output=g)
        np.testing.assert_allclose(out["loss"], c["loss"], rtol=1e-14, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(out["dX"], c["dX"], rtol=1e-14, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(out["dW"], c["dW"], rtol=1e-14, atol=1e-15, err_msg=c["name"])


# ------------------------------------------------------- library routine pin
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("frac", [0.0, 0.3])
def test_against_torch_autograd(oracle_mod, reduction, frac):
    X, W, t = _case(BT=23, H=7, V=11, seed=11, frac=frac)
    g = si.make_grad_output(t, reduction, seed=11, scalar=1.7 if reduction != "none" else 1.0)
    out = oracle_mod.flce(X, W, t, reduction=reduction, grad_output=g)
    l_ref, dx_ref, dw_ref = _torch_ref(X.double().numpy(), W.double().numpy(), t.numpy(),
                                       reduction, g.numpy())
    np.testing.assert_allclose(out["loss"], l_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["dX"], dx_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["dW"], dw_ref, rtol=1e-11, atol=1e-13)


def test_against_torch_ignore_index_inside_vocab(oracle_mod):
    """ignore_index is compared for equality; it may be a valid class id."""
    X, W, _ = _case(BT=17, H=5, V=6, seed=12)
    t = torch.tensor([3, 1, 3, 0, 5, 3, 2, 4, 3, 1, 0, 5, 3, 2, 2, 3, 1])
    out = oracle_mod.flce(X, W, t, ignore_index=3, reduction="mean")
    l_ref, dx_ref, dw_ref = _torch_ref(X.double().numpy(), W.double().numpy(), t.numpy(),
                                       "mean", None, ignore_index=3)
    assert out["n_valid"] == int((t != 3).sum())
    np.testing.assert_allclose(out["loss"], l_ref, rtol=1e-12)
    np.testing.assert_allclose(out["dX"], dx_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["dW"], dw_ref, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------- closed forms
def test_zero_weight_closed_form(oracle_mod):
    BT, H, V = 9, 4, 13
    X, _, t = _case(BT, H, V, seed=13, frac=0.2)
    W = np.zeros((V, H))
    out = oracle_mod.flce(X, W, t, reduction="mean")
    assert out["loss"] == pytest.approx(math.log(V), rel=1e-15)
    assert np.all(out["dX"] == 0.0)
    Xd = X.double().numpy()
    tn = t.numpy()
    lab = tn != -100
    N = lab.sum()
    ref = np.zeros((V, H))
    for i in np.nonzero(lab)[0]:
        ref += (1.0 / N) * (1.0 / V) * Xd[i][None, :]
        ref[tn[i]] -= (1.0 / N) * Xd[i]
    np.testing.assert_allclose(out["dW"], ref, rtol=1e-13, atol=1e-16)


def test_zero_input_closed_form(oracle_mod):
    BT, H, V = 7, 5, 9
    _, W, t = _case(BT, H, V, seed=14, frac=0.3)
    X = np.zeros((BT, H))
    g = si.make_grad_output(t, "none", seed=14)
    out = oracle_mod.flce(X, W, t, reduction="none", grad_output=g)
    tn = t.numpy()
    lab = tn != -100
    np.testing.assert_allclose(out["loss"][lab], math.log(V), rtol=1e-15)
    assert np.all(out["loss"][~lab] == 0.0)
    assert np.all(out["dW"] == 0.0)
    Wd = W.double().numpy()
    gd = g.double().numpy()
    for i in range(BT):
        if lab[i]:
            np.testing.assert_allclose(out["dX"][i], gd[i] * (Wd.mean(0) - Wd[tn[i]]), rtol=1e-12,
                                       atol=1e-15)
        else:
            assert np.all(out["dX"][i] == 0.0)


def test_two_classes_is_softplus(oracle_mod):
    X, W, t = _case(BT=12, H=3, V=2, seed=15)
    out = oracle_mod.flce(X, W, t, reduction="none")
    Z = X.double().numpy() @ W.double().numpy().T
    tn = t.numpy()
    d = Z[np.arange(12), 1 - tn] - Z[np.arange(12), tn]
    np.testing.assert_allclose(out["loss"], np.logaddexp(0.0, d), rtol=1e-14)


# -------------------------------------------------------- finite differences
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_finite_differences(oracle_mod, reduction):
    BT, H, V = 5, 3, 4
    X, W, t = _case(BT, H, V, seed=16, frac=0.2)
    g = si.make_grad_output(t, reduction, seed=16, scalar=0.7)
    Xd = X.double().numpy()
    Wd = W.double().numpy()
    out = oracle_mod.flce(Xd, Wd, t, reduction=reduction, grad_output=g)
    gn = g.double().numpy()
    lab = t.numpy() != -100

    def objective(Xp, Wp):
        o = oracle_mod.flce(Xp, Wp, t, reduction=reduction)
        if reduction == "none":
            return float(np.sum(np.where(lab, o["loss"] * np.nan_to_num(gn), 0.0)))
        return float(o["loss"]) * float(gn[0])

    h = 1e-6
    for arr, grad in ((Xd, out["dX"]), (Wd, out["dW"])):
        fd = np.zeros_like(arr)
        for j in np.ndindex(arr.shape):
            p = arr.copy(); p[j] += h
            m = arr.copy(); m[j] -= h
            if arr is Xd:
                fd[j] = (objective(p, Wd) - objective(m, Wd)) / (2 * h)
            else:
                fd[j] = (objective(Xd, p) - objective(Xd, m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


# ------------------------------------------------------------------ invariants
def test_grad_weight_columns_sum_to_zero(oracle_mod):
    """Rows of softmax - onehot sum to 0, so sum_v dW[v, k] = 0 for every k."""
    X, W, t = _case(BT=31, H=6, V=17, seed=17, frac=0.25)
    out = oracle_mod.flce(X, W, t, reduction="sum")
    colsum = out["dW"].sum(axis=0)
    assert np.max(np.abs(colsum)) < 1e-13 * max(1.0, np.abs(out["dW"]).max() * 17)


def test_common_shift_of_weight_rows(oracle_mod):
    X, W, t = _case(BT=14, H=5, V=8, seed=18, frac=0.2)
    Wd = W.double().numpy()
    c = np.linspace(-0.3, 0.4, 5)
    a = oracle_mod.flce(X, Wd, t, reduction="mean")
    b = oracle_mod.flce(X, Wd + c[None, :], t, reduction="mean")
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(b["dX"], a["dX"], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(b["dW"], a["dW"], rtol=1e-11, atol=1e-14)


def test_block_additivity_is_chunk_invariance(oracle_mod):
    """Any partition of the rows into blocks, some fully ignored, sums to the whole."""
    BT, H, V = 40, 6, 19
    X, W, t = _case(BT, H, V, seed=19)
    t = t.clone()
    t[8:16] = -100  # one fully ignored block
    t[21] = -100
    whole = oracle_mod.flce(X, W, t, reduction="sum")
    bounds = [0, 8, 16, 19, 33, 40]
    loss = 0.0
    dW = np.zeros((V, H))
    dX = np.zeros((BT, H))
    for a, b in zip(bounds[:-1], bounds[1:]):
        part = oracle_mod.flce(X[a:b], W, t[a:b], reduction="sum")
        loss += part["loss"]
        dW += part["dW"]
        dX[a:b] = part["dX"]
    assert loss == pytest.approx(whole["loss"], rel=1e-13)
    np.testing.assert_allclose(dX, whole["dX"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(dW, whole["dW"], rtol=1e-12, atol=1e-15)
    mean = oracle_mod.flce(X, W, t, reduction="mean")
    N = whole["n_valid"]
    assert mean["loss"] == pytest.approx(whole["loss"] / N, rel=1e-13)
    np.testing.assert_allclose(mean["dW"] * N, whole["dW"], rtol=1e-12, atol=1e-15)


def test_reduction_relations(oracle_mod):
    X, W, t = _case(BT=29, H=5, V=10, seed=20, frac=0.3)
    m = oracle_mod.flce(X, W, t, reduction="mean")
    s = oracle_mod.flce(X, W, t, reduction="sum")
    n = oracle_mod.flce(X, W, t, reduction="none")
    N = m["n_valid"]
    assert N == int((t != -100).sum())
    assert s["loss"] == pytest.approx(N * m["loss"], rel=1e-13)
    assert float(np.sum(n["loss"])) == pytest.approx(s["loss"], rel=1e-13)
    np.testing.assert_allclose(s["dX"], N * m["dX"], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(n["dX"], s["dX"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(n["dW"], s["dW"], rtol=1e-12, atol=1e-16)


# ------------------------------------------------------------- ignored rows
def test_ignored_rows_zero_and_nan_isolated(oracle_mod):
    BT, H, V = 24, 5, 9
    X, W, t = _case(BT, H, V, seed=21, frac=0.4)
    g = si.make_grad_output(t, "none", seed=21, nan_at_ignored=False)
    ign = (t == -100).numpy()
    clean = oracle_mod.flce(X, W, t, reduction="none", grad_output=g)
    Xp = X.clone()
    Xp[torch.from_numpy(ign)] = float("nan")
    gp = g.clone()
    gp[torch.from_numpy(ign)] = float("nan")
    pois = oracle_mod.flce(Xp, W, t, reduction="none", grad_output=gp)
    for k in ("loss", "dX", "dW"):
        assert np.array_equal(clean[k], pois[k]), k
    assert np.all(pois["dX"][ign] == 0.0) and not np.signbit(pois["dX"][ign]).any()
    assert np.all(pois["loss"][ign] == 0.0)
    for red in ("mean", "sum"):
        a = oracle_mod.flce(X, W, t, reduction=red)
        b = oracle_mod.flce(Xp, W, t, reduction=red)
        assert a["loss"] == b["loss"]
        assert np.array_equal(a["dX"], b["dX"]) and np.array_equal(a["dW"], b["dW"])


def test_all_rows_ignored(oracle_mod):
    X, W, t = _case(BT=6, H=3, V=5, seed=22, ignore="all")
    for red in ("mean", "sum"):
        o = oracle_mod.flce(X, W, t, reduction=red)
        assert o["loss"] == 0.0 and o["n_valid"] == 0
        assert np.all(o["dX"] == 0.0) and np.all(o["dW"] == 0.0)


def test_compaction_list_and_target_range(oracle_mod):
    t = np.array([5, -100, 0, 3, -100, -100, 9, 1], dtype=np.int64)
    idx, n = oracle_mod.compact(t, V=10)
    assert n == 5 and idx.tolist() == [0, 2, 3, 6, 7]
    with pytest.raises(oracle_mod.OracleTargetError):
        oracle_mod.compact(np.array([0, 10]), V=10)
    with pytest.raises(oracle_mod.OracleTargetError):
        oracle_mod.compact(np.array([0, -1]), V=10)
    idx, n = oracle_mod.compact(np.array([], dtype=np.int64), V=10)
    assert n == 0 and idx.size == 0


def test_accumulate_adds_to_given_weight_grad(oracle_mod):
    X, W, t = _case(BT=10, H=4, V=6, seed=23)
    base = oracle_mod.flce(X, W, t, reduction="sum")
    init = np.linspace(-1, 1, 24).reshape(6, 4)
    acc = oracle_mod.flce(X, W, t, reduction="sum", dW_init=init)
    np.testing.assert_allclose(acc["dW"], init + base["dW"], rtol=1e-15, atol=1e-16)


def test_frozen_weight_skips_grad_weight(oracle_mod):
    X, W, t = _case(BT=10, H=4, V=6, seed=24)
    a = oracle_mod.flce(X, W, t, reduction="sum")
    b = oracle_mod.flce(X, W, t, reduction="sum", frozen=True)
    assert b["dW"] is None
    assert a["loss"] == b["loss"] and np.array_equal(a["dX"], b["dX"])


def test_statistical_band():
    """With X ~ N(0,1), W ~ N(0, 0.02^2): per-row loss has mean ~ ln V + sigma^2/2."""
    import oracle
    BT, H, V = 256, 128, 1024
    X, W, t = si.make_case(BT, H, V, "f32", 1000, ignore="scattered", frac=0.1)
    o = oracle.flce(X, W, t, reduction="mean")
    sigma2 = 4e-4 * H
    assert abs(o["loss"] - (math.log(V) + sigma2 / 2)) < 0.02


# ------------------------------------------------ two implementations agree
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_matmul_variant_matches_loops(oracle_mod, reduction):
    X, W, t = _case(BT=37, H=9, V=21, seed=25, frac=0.3)
    g = si.make_grad_output(t, reduction, seed=25, scalar=1.3)
    a = oracle_mod.flce(X, W, t, reduction=reduction, grad_output=g)
    b = oracle_mod.flce_matmul(X, W, t, reduction=reduction, grad_output=g)
    np.testing.assert_allclose(a["loss"], b["loss"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a["dX"], b["dX"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-12, atol=1e-15)
    lab = t.numpy() != -100
    np.testing.assert_allclose(a["lse"][lab], b["lse"][lab], rtol=1e-14)
    lse_m = oracle_mod.lse_matmul(oracle_mod.widen(X), oracle_mod.widen(W), t, rows_per_block=8)
    lse_l = oracle_mod.lse(X, W, t)
    np.testing.assert_allclose(lse_m[lab], lse_l[lab], rtol=1e-14)
    assert np.all(np.isnan(lse_m[~lab])) and np.all(np.isnan(lse_l[~lab]))


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_matmul_row_subsets_match_loops(oracle_mod, reduction):
    """The matmul forms of the per-row oracle functions (used at full size)
    equal the loop forms on selected rows, ignored ones included."""
    X, W, t = _case(BT=41, H=10, V=19, seed=27, frac=0.3)
    g = si.make_grad_output(t, reduction, seed=27, scalar=1.1)
    Xd, Wd = oracle_mod.widen(X), oracle_mod.widen(W)
    full = oracle_mod.flce(X, W, t, reduction=reduction, grad_output=g)
    N = full["n_valid"]
    rows = np.array([0, 3, 4, 11, 12, 25, 40])
    a = oracle_mod.dx_rows(X, W, t, rows, n_valid=N, reduction=reduction, grad_output=g)
    b = oracle_mod.dx_rows_matmul(Xd, Wd, t, rows, n_valid=N, reduction=reduction,
                                  grad_output=g, rows_per_block=3)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(np.isnan(b[2]), np.isnan(a[2]))
    np.testing.assert_allclose(b[2][~np.isnan(a[2])], a[2][~np.isnan(a[2])], rtol=1e-14)
    np.testing.assert_allclose(b[0], full["dX"][rows], rtol=1e-12, atol=1e-15)
    vrows = np.array([0, 1, 7, 18, int(t[2]) if int(t[2]) >= 0 else 5])
    lse = full["lse"]
    c = oracle_mod.dw_rows(X, W, t, vrows, lse, n_valid=N, reduction=reduction, grad_output=g)
    d = oracle_mod.dw_rows_matmul(Xd, Wd, t, vrows, lse, n_valid=N, reduction=reduction,
                                  grad_output=g, rows_per_block=5)
    np.testing.assert_allclose(d, c, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(d, full["dW"][vrows], rtol=1e-12, atol=1e-15)
    # an ignored X row full of NaN is never read
    Xp = Xd.copy()
    Xp[np.nonzero(t.numpy() == -100)[0]] = np.nan
    e = oracle_mod.dw_rows_matmul(Xp, Wd, t, vrows, lse, n_valid=N, reduction=reduction,
                                  grad_output=g, rows_per_block=5)
    assert e.tobytes() == d.tobytes()


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_row_subsets_match_full(oracle_mod, reduction):
    X, W, t = _case(BT=33, H=8, V=15, seed=26, frac=0.25)
    g = si.make_grad_output(t, reduction, seed=26, scalar=0.9)
    full = oracle_mod.flce(X, W, t, reduction=reduction, grad_output=g)
    rows = np.array([0, 5, 6, 17, 32])
    dx, lr, ls = oracle_mod.dx_rows(X, W, t, rows, n_valid=full["n_valid"], reduction=reduction,
                                    grad_output=g)
    np.testing.assert_array_equal(dx, full["dX"][rows])
    vrows = np.array([0, 3, 14])
    dw = oracle_mod.dw_rows(X, W, t, vrows, full["lse"], n_valid=full["n_valid"],
                            reduction=reduction, grad_output=g)
    np.testing.assert_array_equal(dw, full["dW"][vrows])
    if reduction == "none":
        np.testing.assert_array_equal(lr, full["loss"][rows])


# ------------------------------------------------------------ planted mistakes
MUTANTS = [
    ("onehot sign flipped in grad_input", "(exp(z[v] - l) - (v == ti ? 1.0 : 0.0))",
     "(exp(z[v] - l) + (v == ti ? 1.0 : 0.0))"),
    ("mean divides by the wrong count", "gs / (double)n_valid", "gs / (double)(n_valid + 1)"),
    ("grad_weight uses the wrong operand", "acc[k] += gv * x[k];", "acc[k] += gv * w[k];"),
    ("onehot term dropped from grad_weight", "(exp(z - lse[i]) - (v == t[i] ? 1.0 : 0.0))",
     "(exp(z - lse[i]) - 0.0)"),
    ("loss reads the wrong logit", "lrow[i] = l - z[ti];", "lrow[i] = l - z[0];"),
    ("per-row upstream gradient ignored", "return g ? g[i] : 1.0;", "return g ? g[0] : 1.0;"),
    ("logit index transposed", "acc += w[k] * x[k];", "acc += w[k] * x[k % 2];"),
    ("log dropped from log-sum-exp", "return m + log(s);", "return m + s - 1.0;"),
]


def _pins_pass(oracle_mod) -> bool:
    try:
        test_hand_cases(oracle_mod)
        for red in ("mean", "sum", "none"):
            test_against_torch_autograd(oracle_mod, red, 0.3)
    except AssertionError:
        return False
    return True


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(oracle_mod, tmp_path, name, old, new):
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
        assert not _pins_pass(oracle_mod), f"planted mistake not caught: {name}"
    finally:
        oracle_mod._lib = saved
    assert _pins_pass(oracle_mod)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_loss_from_lse_and_target_logits_match_full_oracle(oracle_mod, reduction):
    """The helpers the full-size GPU tests use reproduce the loop oracle's loss."""
    X, W, t = _case(BT=41, H=7, V=19, seed=27, frac=0.3)
    full = oracle_mod.flce(X, W, t, reduction=reduction)
    Xd, Wd = oracle_mod.widen(X), oracle_mod.widen(W)
    lse = oracle_mod.lse_matmul(Xd, Wd, t)
    zt = oracle_mod.target_logits(Xd, Wd, t)
    got = oracle_mod.loss_from_lse(lse, zt, t, reduction=reduction)
    np.testing.assert_allclose(got, full["loss"], rtol=1e-13, atol=1e-15)
    # and against torch's cross_entropy (library routine)
    l_ref, _, _ = _torch_ref(Xd, Wd, t.numpy(), reduction, None)
    np.testing.assert_allclose(got, l_ref, rtol=1e-12, atol=1e-14)
