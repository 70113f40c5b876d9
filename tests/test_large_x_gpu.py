"""X larger than one 32-bit buffer range (2 GiB): a long-context shape.

PR #1439 (Summary) is about long sequences, where BT x H x itemsize passes
2 GiB: BT 139901 rows of H 8192 in bf16 is 2.29 GB.  The logits GEMM then
reads each chunk's labelled rows gathered into the workspace, a range-sized
block at a time; every other kernel addresses X and dX with 64-bit offsets.

Row i of X is row (i mod 997) of a seeded [997, H] block, so the oracle's
row functions can run on any row cheaply; a 32-bit offset that wrapped at
2 GiB (row 131072 here) would land on a row of another residue and be
caught.  Checks: loss (mean) from the oracle's per-row log-sum-exp, grad_input
on sampled rows on both sides of the 2 GiB boundary and at the end, exact
zeros at ignored rows, grad_weight on sampled vocabulary rows; tolerances
bf16 loss 2e-3, gradients 2e-2 (relative), also per sampled row.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

BT, H, V, P = 139901, 8192, 1000, 997


class _PeriodicRows:
    """Read-only fp64 view of the periodic X: row i is base[i % P]."""

    def __init__(self, base):
        self.base = base
        self.shape = (BT, base.shape[1])

    def __getitem__(self, rows):
        return self.base[np.asarray(rows) % P]


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


def _rows_err(got, ref):
    return np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)


@pytest.mark.parametrize("chunk", [8192, None])
def test_x_over_2gib(pkg, chunk):
    seed = 5151
    base = si.make_x(P, H, "bf16", seed)
    W = si.make_w(V, H, "bf16", seed)
    t = si.make_targets(BT, V, seed, ignore="scattered", frac=0.3)
    assert BT * H * 2 > 2 ** 31
    dev = torch.device("cuda:0")
    print(f"X over 2 GiB: BT={BT} H={H} V={V} bf16 chunk={chunk}", flush=True)
    Xg = base.to(dev)[torch.arange(BT, device=dev) % P].contiguous()
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        Xg, W.to(dev), t.to(dev), reduction="mean", chunk_size=chunk,
        accum_dtype=torch.float32, return_row_index=True)
    torch.cuda.synchronize()
    lab = (t != -100).numpy()
    N = int(lab.sum())
    assert r.stats["n_valid"] == N
    idx_ref, _ = oracle.compact(t, V)
    np.testing.assert_array_equal(r.row_index.cpu().numpy().astype(np.int64), idx_ref)

    Bd, Wd = oracle.widen(base), oracle.widen(W)
    Xd = _PeriodicRows(Bd)
    # loss: the oracle's lse of each distinct row, and target logits per row
    lse_base = oracle.lse_matmul(Bd, Wd, torch.zeros(P, dtype=torch.int64))
    lse = np.where(lab, lse_base[np.arange(BT) % P], np.nan)
    zt = oracle.target_logits(Xd, Wd, t)
    ref_loss = oracle.loss_from_lse(lse, zt, t, reduction="mean")
    assert abs(float(r.loss) - ref_loss) <= 2e-3 * abs(ref_loss)

    # grad_input rows on both sides of the 2 GiB boundary, at the end, and random
    lab_rows = np.nonzero(lab)[0]
    edge = 2 ** 31 // (H * 2)
    rng = np.random.Generator(np.random.PCG64(3))
    near = lab_rows[(lab_rows > edge - 40) & (lab_rows < edge + 40)]
    rows = np.unique(np.concatenate([near, lab_rows[-16:], lab_rows[:4],
                                     rng.choice(lab_rows, 64, replace=False)]))
    dx_ref, _, _ = oracle.dx_rows_matmul(Xd, Wd, t, rows, n_valid=N, reduction="mean")
    dx_got = r.dX[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
    assert _rows_err(dx_got, dx_ref).max() <= 2e-2
    ign = torch.from_numpy(np.nonzero(~lab)[0]).to(dev)
    assert int(r.dX[ign].view(torch.int16).abs().max()) == 0

    # grad_weight rows
    vrows = np.unique(np.concatenate([rng.choice(V, 48, replace=False), [0, V - 1],
                                      t.numpy()[rows[:8]]]))
    vrows = vrows[vrows >= 0]
    dw_ref = oracle.dw_rows_matmul(Xd, Wd, t, vrows, lse, n_valid=N, reduction="mean")
    dw_got = r.dW[torch.from_numpy(vrows).to(dev)].double().cpu().numpy()
    errs = _rows_err(dw_got, dw_ref)
    print(f"dX worst row {_rows_err(dx_got, dx_ref).max():.2e}, dW worst row {errs.max():.2e}",
          flush=True)
    assert errs.max() <= 2e-2
