"""Seeded random configurations of the differentiable entries (the
autograd.Function wrapper and the torch custom op) against the oracle.

Each case draws the operand dtype, the shape, the chunk size, the reduction,
a bias, a z-loss coefficient, fp32 or weight-dtype accumulation, a frozen
weight, an ignored share with -100 or an ignore_index inside [0, V), and a
random upstream gradient (per token for none, with NaN at ignored rows, which
backward must never read).  loss.backward() must give x.grad, weight.grad and
bias.grad in the inputs' dtypes, matching the oracle's gradients to the usual
tolerances (fp32 loss 1e-5, gradients 1e-4; 16-bit 2e-3 and 2e-2), with
exact zeros in the ignored rows of x.grad.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2), "f16": (2e-3, 2e-2)}
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
N_CASES = 48


def draw(i):
    """The configuration of case i (a pure function of i)."""
    r = np.random.Generator(np.random.PCG64(4242 + i))
    pick = lambda xs: xs[int(r.integers(len(xs)))]
    V = int(pick([2, int(r.integers(3, 200)), int(r.integers(200, 900))]))
    return dict(entry=pick(["wrapper", "op"]), dtype=pick(["f32", "bf16", "f16"]),
                BT=int(pick([1, int(r.integers(2, 80)), int(r.integers(80, 300))])),
                H=8 * int(r.integers(1, 17)), V=V,
                chunk=pick([None, 16, 64, 100, 256]),
                reduction=pick(["mean", "sum", "none"]),
                bias=bool(r.random() < 0.5), lam=float(pick([0.0, 1e-3])),
                accum_fp32=bool(r.random() < 0.5), frozen=bool(r.random() < 0.2),
                ignore=pick(["none", "scattered", "prompt_first"]),
                frac=float(pick([0.2, 0.6])),
                ignore_index=-100 if r.random() < 0.7 else int(r.integers(0, V)),
                scalar=float(pick([1.0, 0.3, 2.5])), seed=9000 + 11 * i)


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


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_differentiable_call(pkg, i):
    c = draw(i)
    dt, BT, H, V, ii, red = c["dtype"], c["BT"], c["H"], c["V"], c["ignore_index"], c["reduction"]
    print(f"case {i}: {c}", flush=True)
    X = si.make_x(BT, H, dt, c["seed"])
    W = si.make_w(V, H, dt, c["seed"], scale=0.5 if dt == "f32" else 0.1)
    t = si.make_targets(BT, V, c["seed"], ignore=c["ignore"], frac=c["frac"], ignore_index=ii)
    lab = (t != ii).numpy()
    b = (si.make_x(1, V, "f32", c["seed"] + 7).reshape(-1) * 0.5).to(TD[dt]) if c["bias"] else None
    g = si.make_grad_output(t, red, c["seed"], scalar=c["scalar"], ignore_index=ii)

    dev = torch.device("cuda:0")
    x = X.to(dev).requires_grad_(True)
    w = W.to(dev).requires_grad_(not c["frozen"])
    bb = None if b is None else b.to(dev).requires_grad_(True)
    if c["entry"] == "wrapper":
        loss = pkg.fused_linear_cross_entropy(
            x, w, t.to(dev), bb, ignore_index=ii, reduction=red, chunk_size=c["chunk"],
            accum_dtype=torch.float32 if c["accum_fp32"] else None, z_loss_scale=c["lam"])
    else:
        loss = pkg.fused_linear_cross_entropy_op(
            x, w, t.to(dev), bb, ignore_index=ii, reduction=red, chunk_size=c["chunk"] or 0,
            accum_fp32=c["accum_fp32"], z_loss_scale=c["lam"])
    loss.backward(g.to(dev) if red == "none" else g.to(dev).reshape(()))
    torch.cuda.synchronize()

    ref = oracle.flce_ex(X, W, t, bias=b, z_loss_scale=c["lam"], ignore_index=ii, reduction=red,
                         grad_output=torch.nan_to_num(g).numpy())
    tl, tg = TOL[dt]
    if red == "none":
        lo = loss.detach().cpu().numpy()
        assert np.all(lo[~lab] == 0.0)
        if lab.any():
            assert _rel(lo[lab], ref["loss"][lab]) <= tl
    elif lab.any():
        assert abs(float(loss) - ref["loss"]) <= tl * max(abs(ref["loss"]), 1e-30)
    else:
        assert float(loss) == 0.0

    assert x.grad.dtype == TD[dt]
    gx = x.grad.float().cpu().numpy()
    assert np.all(gx[~lab] == 0.0)
    assert _rel(gx, ref["dX"]) <= tg
    if c["frozen"]:
        assert w.grad is None
    else:
        assert w.grad.dtype == TD[dt]
        assert _rel(w.grad.double().cpu().numpy(), ref["dW"]) <= tg
    if b is not None:
        assert bb.grad.dtype == TD[dt]
        assert _rel(bb.grad.double().cpu().numpy(), ref["grad_bias"]) <= tg
