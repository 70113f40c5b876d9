"""GPU parity at the full benchmark sizes, in the launch configurations bench.py times.

The oracle cannot run every output element at these sizes, so each case checks:
* the loss (mean / sum) against the oracle's exact value, from the stored
  per-row log-sum-exp (tests/golden/full_size/*.npz, written by
  make_full_size_lse.py with the oracle only) and the oracle's target logits;
* grad_input on sampled rows and grad_weight on sampled vocabulary rows
  (including some targets), computed one by one by the oracle;
* per-row losses on sampled rows for reduction none, and exact zeros at
  ignored rows;
* sum over the vocabulary of grad_weight ~ 0 (rows of softmax - onehot sum
  to zero), a property that holds at any size.
Tolerances: fp32 loss 1e-5, gradients 1e-4; bf16/fp16 loss 2e-3, gradients
2e-2 (relative Frobenius over the sample).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden", "full_size")
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2), "f16": (2e-3, 2e-2)}
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# (case id, golden set, BT used, chunk_size, accum, reduction, labelled share, frozen[,
#  sequence length of the packed sequences; default one sequence of BT])
CASES = [
    ("llama_c2048", "llama3_8b_lm_head", 8192, 2048, "f32", "mean", 1.0, False),
    ("llama_c256", "llama3_8b_lm_head", 8192, 256, "f32", "mean", 1.0, False),
    ("sweep_bf16", "same_dtype_sweep_bf16", 16384, 0, "same", "mean", 1.0, False),
    ("sweep_f16", "same_dtype_sweep_f16", 16384, 0, "same", "mean", 1.0, False),
    ("sweep_f32", "same_dtype_sweep_f32", 16384, 0, "same", "mean", 1.0, False),
    ("longseq_8k_c256", "long_seq_large_vocab", 8192, 256, "same", "mean", 1.0, False),
    ("longseq_8k_default", "long_seq_large_vocab", 8192, 0, "same", "mean", 1.0, False),
    ("longseq_32k_c256", "long_seq_large_vocab", 32768, 256, "same", "mean", 1.0, False),
    ("longseq_32k_default", "long_seq_large_vocab", 32768, 0, "same", "mean", 1.0, False),
    ("sft_100_trained_sum", "masked_sft", 8192, 0, "same", "sum", 1.0, False),
    ("sft_75_trained_sum", "masked_sft", 8192, 0, "same", "sum", 0.75, False),
    ("sft_50_trained_sum", "masked_sft", 8192, 0, "same", "sum", 0.5, False),
    ("sft_10_trained_sum", "masked_sft", 8192, 0, "same", "sum", 0.1, False),
    ("sft_75_frozen_none", "masked_sft", 8192, 0, "same", "none", 0.75, True),
    ("sft_10_frozen_none", "masked_sft", 8192, 0, "same", "none", 0.1, True),
    ("sft_50_packed_trained_sum", "masked_sft", 8192, 0, "same", "sum", 0.5, False, 1024),
    ("sft_75_packed_frozen_none", "masked_sft", 8192, 0, "same", "none", 0.75, True, 1024),
]

_cache = {}


def _inputs(gset, BT):
    """Host inputs of a golden set (cached; the BT-row prefix when smaller)."""
    if gset not in _cache:
        _cache.clear()
        g = np.load(os.path.join(GOLD, gset + ".npz"))
        BTg, H, V, dt, seed = int(g["BT"]), int(g["H"]), int(g["V"]), str(g["dtype"]), int(g["seed"])
        X = si.make_x(BTg, H, dt, seed)
        W = si.make_w(V, H, dt, seed)
        t = si.make_targets(BTg, V, seed)
        _cache[gset] = dict(X=X, W=W, t=t, lse=g["lse"], dt=dt, seed=seed,
                            Xd=oracle.widen(X), Wd=oracle.widen(W))
    c = _cache[gset]
    return c, BT


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_full_size(pkg, case):
    cid, gset, BT, chunk, accum, red, share, frozen = case[:8]
    seq = case[8] if len(case) > 8 else BT
    c, BT = _inputs(gset, BT)
    dt = c["dt"]
    tl, tg = TOL[dt]
    X, W = c["X"][:BT], c["W"]
    t = c["t"][:BT].clone()
    if share < 1.0:  # masked SFT: the first (1 - share) of each sequence is ignored
        for s0 in range(0, BT, seq):
            t[s0:s0 + int(round((1.0 - share) * min(seq, BT - s0)))] = -100
    Xd, Wd = c["Xd"][:BT], c["Wd"]
    lse = c["lse"][:BT].copy()
    lab = (t != -100).numpy()
    lse[~lab] = np.nan
    N = int(lab.sum())
    g = si.make_grad_output(t, red, c["seed"], scalar=1.0) if red == "none" else None
    print(f"[{cid}] BT={BT} H={X.shape[1]} V={W.shape[0]} {dt} chunk={chunk} {red} "
          f"share={share} seq={seq} frozen={frozen}", flush=True)

    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), reduction=red, chunk_size=chunk or None,
        accum_dtype=torch.float32 if accum == "f32" else None, frozen_weight=frozen,
        grad_output=None if g is None else g.to(dev))
    torch.cuda.synchronize()
    assert r.stats["n_valid"] == N

    # loss
    zt = oracle.target_logits(Xd, Wd, t)
    ref_loss = oracle.loss_from_lse(lse, zt, t, reduction=red)
    if red == "none":
        got = r.loss.cpu().numpy()
        assert np.all(got[~lab] == 0.0)
        loss_err = _rel(got[lab], ref_loss[lab])
    else:
        loss_err = abs(float(r.loss) - ref_loss) / abs(ref_loss)
    assert loss_err <= tl, loss_err

    # sampled grad_input rows
    rng = np.random.Generator(np.random.PCG64(7))
    lab_rows = np.nonzero(lab)[0]
    rows = np.unique(np.concatenate([rng.choice(lab_rows, 14, replace=False),
                                     lab_rows[[0, -1]]]))
    if not lab.all():
        rows = np.concatenate([rows, np.nonzero(~lab)[0][:2]])
    dx_ref, lrow, _ = oracle.dx_rows(Xd, Wd, t, rows, n_valid=N, reduction=red, grad_output=g)
    dx_got = r.dX[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
    dx_err = _rel(dx_got, dx_ref)
    assert dx_err <= tg, dx_err
    ign = ~lab[rows]
    assert np.all(dx_got[ign] == 0.0)
    if red == "none":
        assert _rel(r.loss.cpu().numpy()[rows][~ign], lrow[~ign]) <= tl

    # sampled grad_weight rows (some random, some that are targets)
    if not frozen:
        V = W.shape[0]
        vrows = np.unique(np.concatenate([rng.choice(V, 12, replace=False),
                                          t.numpy()[rows[:4]]]))
        vrows = vrows[vrows >= 0]
        dw_ref = oracle.dw_rows(Xd, Wd, t, vrows, lse, n_valid=N, reduction=red, grad_output=g)
        dw_got = r.dW[torch.from_numpy(vrows).to(dev)].double().cpu().numpy()
        dw_err = _rel(dw_got, dw_ref)
        assert dw_err <= tg, dw_err
        colsum = r.dW.double().sum(0)
        scale = r.dW.double().abs().sum(0)
        assert float((colsum.abs() / scale.clamp_min(1e-30)).max()) <= 5e-2
    else:
        dw_err = float("nan")
    print(f"[{cid}] rel errors: loss {loss_err:.2e}  dX {dx_err:.2e}  dW {dw_err:.2e}", flush=True)
