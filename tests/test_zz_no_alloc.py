"""The no-allocation entry point (flce_fwd_bwd_ex_noalloc) against
flce_fwd_bwd_ex, through the C ABI.

Both run the same kernels; the no-allocation entry point takes its workspace
from the library's static per-GPU scratch instead of an argument.  Two calls
in a row on one GPU share that scratch, the second with a smaller input, and
each must give exactly (bit for bit) the outputs of flce_fwd_bwd_ex on the
same inputs, and match the oracle within the tolerances of the other parity
tests (fp32 loss 1e-5, gradients 1e-4; bf16 loss 2e-3, gradients 2e-2).
The call must not allocate through torch either.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2)}


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _call(pkg, noalloc, X, W, t, b, dt, red, chunk, g, lam):
    """One call through the C ABI; outputs preallocated here."""
    dev = X.device
    BT, H = X.shape
    V = W.shape[0]
    code = pkg.F32 if dt == "f32" else pkg.BF16
    nout = BT if red == "none" else 1
    loss = torch.empty(nout, dtype=torch.float32, device=dev)
    dX = torch.empty_like(X)
    dW = torch.empty(V, H, dtype=torch.float32, device=dev)
    db = torch.empty(V, dtype=torch.float32, device=dev)
    zl = torch.empty(nout, dtype=torch.float32, device=dev)
    acc = torch.empty(nout, dtype=torch.float32, device=dev)
    pred = torch.empty(BT, dtype=torch.int64, device=dev)
    opt = pkg.FlceOptions(0, b.data_ptr(), db.data_ptr(), lam, zl.data_ptr(), acc.data_ptr(),
                          pred.data_ptr())
    st = pkg.FlceStats()
    stream = torch.cuda.current_stream(dev).cuda_stream
    red_code = pkg.REDUCTIONS[red]
    gp = g.data_ptr() if g is not None else None
    args = (X.data_ptr(), W.data_ptr(), t.data_ptr(), BT, H, V, code, -100, red_code, chunk, 1,
            pkg.F32, 0, 0, gp, loss.data_ptr(), dX.data_ptr(), dW.data_ptr())
    torch.cuda.synchronize()
    if noalloc:
        before = torch.cuda.memory_allocated(dev)
        rc = pkg.flce_fwd_bwd_ex_noalloc(*args, stream, st, opt)
        assert torch.cuda.memory_allocated(dev) == before
    else:
        need = pkg.flce_workspace_bytes_ex(BT, H, V, code, chunk, 1, opt)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        rc = pkg.flce_fwd_bwd_ex(*args, ws.data_ptr(), need, stream, st, opt)
    assert rc == 0, (rc, pkg.flce_last_error())
    torch.cuda.synchronize()
    return dict(loss=loss, dX=dX, dW=dW, grad_bias=db, z_loss=zl, accuracy=acc, predicted=pred), \
        st.as_dict()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("red", ["mean", "none"])
def test_noalloc_matches_workspace_entry(pkg, dt, red):
    dev = torch.device("cuda:0")
    # the first call fills much of the scratch; the second, smaller one reuses it
    for BT, H, V, chunk, seed in [(700, 256, 3000, 256, 61), (130, 64, 500, 64, 62)]:
        print(f"noalloc {dt} {red}: BT={BT} H={H} V={V} chunk={chunk}", flush=True)
        X = si.make_x(BT, H, dt, seed)
        W = si.make_w(V, H, dt, seed, scale=0.5 if dt == "f32" else 0.1)
        t = si.make_targets(BT, V, seed, ignore="scattered", frac=0.2)
        b = (si.make_x(1, V, "f32", seed + 7).reshape(-1) * 0.5).to(TD[dt])
        g = si.make_grad_output(t, red, seed, scalar=0.75)
        Xg, Wg, tg_, bg = X.to(dev), W.to(dev), t.to(dev), b.to(dev)
        gg = g.to(dev)
        lam = 1e-3
        got, st_a = _call(pkg, True, Xg, Wg, tg_, bg, dt, red, chunk, gg, lam)
        ref, st_b = _call(pkg, False, Xg, Wg, tg_, bg, dt, red, chunk, gg, lam)
        assert st_a == st_b
        for k in ref:
            assert got[k].view(torch.uint8).equal(ref[k].view(torch.uint8)), k
        o = oracle.flce_ex(X, W, t, bias=b, z_loss_scale=lam, reduction=red,
                           grad_output=torch.nan_to_num(g).numpy())
        tl, tgr = TOL[dt]
        lab = (t != -100).numpy()
        if red == "none":
            assert _rel(got["loss"].cpu().numpy()[lab], o["loss"][lab]) <= tl
        else:
            assert abs(float(got["loss"][0]) - o["loss"]) <= tl * abs(o["loss"])
        assert _rel(got["dX"].double().cpu(), o["dX"]) <= tgr
        assert _rel(got["dW"].double().cpu(), o["dW"]) <= tgr
        assert _rel(got["grad_bias"].double().cpu(), o["grad_bias"]) <= tgr


def test_noalloc_refuses_oversized_call(pkg):
    """Beyond the static scratch: FLCE_E_WORKSPACE before any launch, outputs untouched."""
    dev = torch.device("cuda:0")
    BT, H, V = 2048, 4096, 64000  # a chunk of 2048 rows needs about 346 MiB
    X = torch.zeros(BT, H, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(V, H, dtype=torch.bfloat16, device=dev)
    t = torch.zeros(BT, dtype=torch.int64, device=dev)
    loss = torch.full((1,), 7.0, device=dev)
    dX = torch.full((BT, H), 3.0, dtype=torch.bfloat16, device=dev)
    assert pkg.flce_workspace_bytes(BT, H, V, pkg.BF16, 2048, 1) > pkg.SCRATCH_BYTES
    rc = pkg.flce_fwd_bwd_ex_noalloc(X.data_ptr(), W.data_ptr(), t.data_ptr(), BT, H, V,
                                     pkg.BF16, -100, pkg.MEAN, 2048, 1, pkg.BF16, 1, 0, None,
                                     loss.data_ptr(), dX.data_ptr(), None,
                                     torch.cuda.current_stream(dev).cuda_stream, None, None)
    torch.cuda.synchronize()
    assert rc == -4
    assert float(loss[0]) == 7.0 and bool((dX == 3.0).all())
