"""The differentiable entries on the GPU: the autograd.Function wrapper and the
torch custom op, eager and under torch.compile, against the oracle.

For each reduction, with bias and a z-loss coefficient, the loss and the
gradients of x, weight and bias for a random upstream gradient are compared
with oracle.flce_ex (fp32: loss 1e-5, gradients 1e-4 relative).  The none
reduction runs a loss-only forward and re-enters in backward; mean and sum
scale the forward's gradients.  torch.compile(fullgraph=True) must keep the
op opaque and reproduce eager bit for bit; torch.library.opcheck checks the
op's schema, fake implementation and autograd registration.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


def _case(seed=41, BT=150, H=64, V=333):
    X = si.make_x(BT, H, "f32", seed)
    W = si.make_w(V, H, "f32", seed, scale=0.5)
    t = si.make_targets(BT, V, seed, ignore="scattered", frac=0.2)
    b = si.make_x(1, V, "f32", seed + 7).reshape(-1) * 0.5
    return X, W, t, b


def _run(fn, X, W, t, b, reduction, g):
    dev = torch.device("cuda:0")
    x = X.to(dev).requires_grad_(True)
    w = W.to(dev).requires_grad_(True)
    bb = b.to(dev).requires_grad_(True)
    loss = fn(x, w, t.to(dev), bb, reduction)
    loss.backward(g.to(dev) if reduction == "none" else g.to(dev).reshape(()))
    torch.cuda.synchronize()
    return loss.detach(), x.grad, w.grad, bb.grad


def _wrapper(pkg, lam):
    return lambda x, w, t, b, red: pkg.fused_linear_cross_entropy(
        x, w, t, b, reduction=red, chunk_size=64, z_loss_scale=lam)


def _op(pkg, lam):
    return lambda x, w, t, b, red: pkg.fused_linear_cross_entropy_op(
        x, w, t, b, reduction=red, chunk_size=64, z_loss_scale=lam)


@pytest.mark.parametrize("entry", ["wrapper", "op"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_differentiable_entries_match_oracle(pkg, entry, reduction):
    X, W, t, b = _case()
    lam = 2e-3
    if reduction == "none":
        g = si.make_grad_output(t, "none", 41, scalar=1.0)
        g = torch.where(t != -100, g, torch.zeros_like(g))
    else:
        g = torch.tensor([1.7])
    fn = (_wrapper if entry == "wrapper" else _op)(pkg, lam)
    loss, gx, gw, gb = _run(fn, X, W, t, b, reduction, g)
    ref = oracle.flce_ex(X, W, t, bias=b, z_loss_scale=lam, reduction=reduction,
                         grad_output=g.numpy() if reduction == "none" else g.numpy())
    if reduction == "none":
        assert _rel(loss.cpu(), ref["loss"]) <= 1e-5
    else:
        assert abs(float(loss) - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    assert _rel(gx.cpu(), ref["dX"]) <= 1e-4
    assert _rel(gw.cpu(), ref["dW"]) <= 1e-4
    assert _rel(gb.cpu(), ref["grad_bias"]) <= 1e-4


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_compiled_op_matches_eager(pkg, reduction):
    X, W, t, b = _case(seed=3)
    g = torch.ones(X.shape[0]) if reduction == "none" else torch.tensor([1.0])

    def f(x, w, t_, b_, red):
        return pkg.fused_linear_cross_entropy_op(x, w, t_, b_, reduction=red, chunk_size=64)

    eager = _run(f, X, W, t, b, reduction, g)
    torch._dynamo.reset()
    compiled = torch.compile(f, fullgraph=True, dynamic=False)
    comp = _run(compiled, X, W, t, b, reduction, g)
    for a, c in zip(eager, comp):
        assert torch.equal(a, c)


def test_opcheck(pkg):
    X, W, t, b = _case(seed=8, BT=70, H=32, V=130)
    dev = torch.device("cuda:0")
    args = (X.to(dev).requires_grad_(True), W.to(dev).requires_grad_(True), t.to(dev),
            b.to(dev).requires_grad_(True), -100, "mean", 32, 1, True, False, 0.0, True)
    torch.library.opcheck(torch.ops.flce.fused_linear_cross_entropy.default, args,
                          test_utils=("test_schema", "test_faketensor",
                                      "test_autograd_registration"))
    gargs = (X.to(dev), W.to(dev), t.to(dev), b.to(dev), torch.ones(70, device=dev), -100, "none",
             32, 1, True, False, 0.0)
    torch.library.opcheck(torch.ops.flce.fused_linear_cross_entropy_backward.default, gargs,
                          test_utils=("test_schema", "test_faketensor"))


@pytest.mark.parametrize("entry", ["wrapper", "op"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_retained_graph_backward_twice(pkg, entry, reduction, dtype):
    """Two backward passes through one retained graph, upstream gradient 2.0:
    both give the oracle's gradients for that upstream gradient.  Backward must
    not scale the tensors the forward saved (PR #1554, Tests: the none
    reduction re-enters with reusable buffers; mean and sum keep the
    forward's gradients), and the gradients it returns must not share
    storage with them."""
    X, W, t, b = _case(seed=23)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    X, W, b = X.to(td), W.to(td), b.to(td)
    dev = torch.device("cuda:0")
    fn = (_wrapper if entry == "wrapper" else _op)(pkg, 0.0)
    x = X.to(dev).requires_grad_(True)
    w = W.to(dev).requires_grad_(True)
    bb = b.to(dev).requires_grad_(True)
    loss = fn(x, w, t.to(dev), bb, reduction)
    if reduction == "none":
        g = torch.where(t != -100, torch.full(t.shape, 2.0), torch.zeros(t.shape))
    else:
        g = torch.tensor([2.0])
    gd = g.to(dev) if reduction == "none" else g.to(dev).reshape(())
    ref = oracle.flce_ex(X, W, t, bias=b, reduction=reduction, grad_output=g.numpy())
    tg = 1e-4 if dtype == "f32" else 2e-2
    grads = []
    for _ in range(2):
        x.grad = w.grad = bb.grad = None
        loss.backward(gd, retain_graph=True)
        torch.cuda.synchronize()
        grads.append((x.grad.clone(), w.grad.clone(), bb.grad.clone()))
        assert _rel(x.grad.double().cpu(), ref["dX"]) <= tg
        assert _rel(w.grad.double().cpu(), ref["dW"]) <= tg
        assert _rel(bb.grad.double().cpu(), ref["grad_bias"]) <= tg
        # writing into the returned gradients must not reach the saved state
        x.grad.mul_(100.0)
        w.grad.mul_(100.0)
        bb.grad.mul_(100.0)
    for a, c in zip(grads[0], grads[1]):
        assert torch.equal(a, c)
