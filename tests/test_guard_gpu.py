"""Nothing is written outside the caller's output buffers, and the inputs are
left untouched.

The loss, dX, dW and the workspace are each carved out of a larger device
buffer whose bytes before and after the region hold a fixed pattern; after a
call through the C ABI every guard byte must be unchanged.  The cases cover
every tile path (eight-wave and four-wave 256 x 256, 128 x 128), ragged edges
in every dimension, grad_input split over V, the none reduction and a frozen
weight.  The results themselves are checked against the oracle elsewhere; here
only the loss is, so that a passing case has also computed something.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side of a region (keeps 256-byte alignment)
PAT = 0xA5
ITEM = {"f32": 4, "bf16": 2, "f16": 2}

# dtype, BT, H, V, chunk, accum, reduction, frozen
CASES = [
    ("bf16", 900, 392, 1100, 512, "f32", "mean", False),
    ("bf16", 300, 136, 1001, 64, "same", "none", False),
    ("f32", 300, 256, 1000, 64, "f32", "sum", False),
    ("f32", 900, 392, 1100, 512, "f32", "sum", False),
    ("f16", 64, 256, 8192, 64, "f32", "mean", False),
    ("bf16", 200, 128, 900, 32, "same", "sum", True),
]


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


class Guarded:
    def __init__(self, nbytes, dev):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * GUARD,), PAT, dtype=torch.uint8, device=dev)

    @property
    def ptr(self):
        return self.buf.data_ptr() + GUARD

    def intact(self):
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:GUARD] == PAT) and np.all(b[GUARD + self.n:] == PAT))


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-c{c[4]}-{c[6]}"
                                             + ("-frozen" if c[7] else "") for c in CASES])
def test_writes_stay_inside_buffers(pkg, case):
    dtype, BT, H, V, chunk, accum, red, frozen = case
    dev = torch.device("cuda:0")
    X, W, t = si.make_case(BT, H, V, dtype, 2800 + BT, ignore="scattered", frac=0.15)
    g = si.make_grad_output(t, red, 2800, scalar=1.0) if red == "none" else None
    dt = {"f32": pkg.F32, "f16": pkg.F16, "bf16": pkg.BF16}[dtype]
    adt = pkg.F32 if accum == "f32" else dt
    a_item = 4 if accum == "f32" else ITEM[dtype]
    Xd, Wd, td = X.to(dev), W.to(dev), t.to(dev)
    gd = None if g is None else g.to(dev)

    loss = Guarded(4 * (BT if red == "none" else 1), dev)
    dX = Guarded(BT * H * ITEM[dtype], dev)
    dW = None if frozen else Guarded(V * H * a_item, dev)
    wsb = pkg.flce_workspace_bytes(BT, H, V, dt, chunk, 1)
    ws = Guarded(wsb, dev)
    st = pkg.FlceStats()
    rc = pkg.flce_fwd_bwd(Xd.data_ptr(), Wd.data_ptr(), td.data_ptr(), BT, H, V, dt, -100,
                          pkg.REDUCTIONS[red], chunk, 1, adt, int(frozen), 0,
                          None if gd is None else gd.data_ptr(), loss.ptr, dX.ptr,
                          None if dW is None else dW.ptr, ws.ptr, wsb,
                          torch.cuda.current_stream(dev).cuda_stream, st)
    torch.cuda.synchronize()
    assert rc == 0, pkg.flce_status_string(rc)
    # inputs are read only
    assert torch.equal(Xd.cpu(), X) and torch.equal(Wd.cpu(), W) and torch.equal(td.cpu(), t)
    for name, b in (("loss", loss), ("dX", dX), ("dW", dW), ("workspace", ws)):
        if b is not None:
            assert b.intact(), f"{name} guard bytes overwritten"

    got = loss.buf[GUARD:GUARD + loss.n].view(torch.float32).cpu().numpy()
    ref = oracle.flce(X, W, t, reduction=red, frozen=frozen,
                      grad_output=None if g is None else torch.nan_to_num(g))
    tol = 1e-5 if dtype == "f32" else 2e-3
    if red == "none":
        lab = (t != -100).numpy()
        d = np.linalg.norm(got[lab] - ref["loss"][lab]) / np.linalg.norm(ref["loss"][lab])
        assert d <= tol and np.all(got[~lab] == 0.0)
    else:
        assert abs(float(got[0]) - ref["loss"]) <= tol * abs(ref["loss"])
