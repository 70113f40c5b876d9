"""GPU parity at the full benchmark sizes, in the launch configurations bench.py times.

The oracle cannot run every output element at these sizes, so each case checks:
* the inputs regenerate to the fingerprint stored with the golden values;
* the labelled-row index the call built (int32, read back from its
  workspace) equals the oracle's compaction bit for bit (PR #1554, Summary:
  nonzero() of the mask gives the rows), and n_valid with it;
* the loss (mean / sum) against the oracle's exact value, from the stored
  per-row log-sum-exp (tests/golden/full_size/*.npz, written by
  make_full_size_lse.py with the oracle only) and the oracle's target logits;
* grad_input on at least 128 random labelled rows plus fixed picks: the first
  and last labelled row of every chunk, and rows of the last, ragged 256-row
  tile of the last chunk.  Each sampled row sums over every vocabulary split
  of the grad_input reduction;
* grad_weight on at least 128 random vocabulary rows plus fixed picks: every
  row of the last 256-row tile over the vocabulary (the ragged one at
  V = 151936), rows on both sides of each grad_input split boundary over V,
  the first and last row, and some targets;
* every sampled row's own relative error within the tolerance, and the
  relative Frobenius error over the sample (for an fp16 grad_weight the
  per-row check first allows the absolute error fp16's subnormal spacing
  imposes on tiny values, see _storage_floor);
* exact +0.0 (sign bit clear) in every ignored row of grad_input, and of the
  per-token loss for reduction none; per-row losses on the sampled rows;
* sum over the vocabulary of grad_weight ~ 0 (rows of softmax - onehot sum
  to zero), a property that holds at any size.
The sampled rows are computed one by one by the oracle's matmul forms of its
per-row functions (pinned to the loop forms in test_oracle_pins.py).
Tolerances: fp32 loss 1e-5, gradients 1e-4; bf16/fp16 loss 2e-3, gradients
2e-2 (relative).
"""
import importlib.util
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
N_RANDOM = 128

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


def _fingerprint_fn():
    spec = importlib.util.spec_from_file_location(
        "make_full_size_lse", os.path.join(os.path.dirname(__file__), "golden",
                                           "make_full_size_lse.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.fingerprint


def _inputs(gset):
    """Host inputs of a golden set (cached), checked against the stored fingerprint."""
    if gset not in _cache:
        _cache.clear()
        g = np.load(os.path.join(GOLD, gset + ".npz"))
        BTg, H, V, dt, seed = int(g["BT"]), int(g["H"]), int(g["V"]), str(g["dtype"]), int(g["seed"])
        X = si.make_x(BTg, H, dt, seed)
        W = si.make_w(V, H, dt, seed)
        t = si.make_targets(BTg, V, seed)
        fp = _fingerprint_fn()(X, W, t)
        assert fp == str(g["fingerprint"]), (
            f"{gset}: regenerated inputs do not match the stored golden values "
            f"({fp} != {g['fingerprint']}); rerun tests/golden/make_full_size_lse.py")
        _cache[gset] = dict(X=X, W=W, t=t, lse=g["lse"], dt=dt, seed=seed,
                            Xd=oracle.widen(X), Wd=oracle.widen(W))
    return _cache[gset]


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _row_errors(got, ref, floor=0.0):
    """Per-row relative error; `floor` is an absolute error per element that the
    storage format itself imposes, charged as sqrt(H) * floor to the row."""
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    return np.maximum(num - np.sqrt(ref.shape[1]) * floor, 0.0) / den


def _storage_floor(dtype, accum, chunks):
    """Absolute error per element a 16-bit grad_weight cannot avoid: fp16's
    smallest (subnormal) spacing is 2^-24, so each of the `chunks` roundings
    of an accumulated value may err by half of it, however small the value;
    independent roundings add up like sqrt(chunks).  (A wrong row, with an
    error as large as the row, still fails: the allowance is about a third
    of such a row's norm here.)
    Vocabulary rows that no labelled row targets hold mean-reduced gradients
    of order 1/(V N) (about 2e-7 at N 16384, V 32000), a few such spacings,
    where fp16 keeps only a few bits.  bf16 and fp32 share fp32's exponent
    range, and their subnormal spacing (2^-133, 2^-149) is negligible here."""
    if accum == "same" and dtype == "f16":
        return np.sqrt(chunks) * 2.0 ** -25
    return 0.0


def _dx_picks(lab_rows, chunk, rng):
    """Random labelled rows, first / last labelled row of every chunk, and rows
    of the last chunk's ragged 256-row tile."""
    N = lab_rows.size
    n_chunks = -(-N // chunk)
    picks = [rng.choice(lab_rows, min(N_RANDOM, N), replace=False)]
    ends = []
    for k in range(n_chunks):
        ends += [k * chunk, min((k + 1) * chunk, N) - 1]
    picks.append(lab_rows[np.array(ends, dtype=np.int64)])
    last = (n_chunks - 1) * chunk
    tail0 = last + ((N - last) // 256) * 256  # first row of the last, ragged row tile
    if tail0 < N:
        picks.append(lab_rows[np.unique(np.linspace(tail0, N - 1, 8).astype(np.int64))])
    return np.unique(np.concatenate(picks))


def _dw_picks(V, splits_k, t_rows, rng):
    """Random vocabulary rows, the last 256-row tile, both sides of each
    grad_input split boundary over V, the first and last row, and targets."""
    picks = [rng.choice(V, min(N_RANDOM, V), replace=False),
             np.arange(((V - 1) // 256) * 256, V), np.array([0, V - 1]), t_rows]
    for b in splits_k:
        if 0 < b < V:
            picks.append(np.array([b - 1, b]))
    v = np.unique(np.concatenate(picks).astype(np.int64))
    return v[(v >= 0) & (v < V)]


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_full_size(pkg, case):
    cid, gset, BT, chunk, accum, red, share, frozen = case[:8]
    seq = case[8] if len(case) > 8 else BT
    c = _inputs(gset)
    dt = c["dt"]
    tl, tg = TOL[dt]
    X, W = c["X"][:BT], c["W"]
    t = c["t"][:BT].clone()
    if share < 1.0:  # masked SFT: the first (1 - share) of each sequence is ignored
        for s0 in range(0, BT, seq):
            t[s0:s0 + int(round((1.0 - share) * min(seq, BT - s0)))] = -100
    Xd, Wd = c["Xd"][:BT], c["Wd"]
    H, V = X.shape[1], W.shape[0]
    lse = c["lse"][:BT].copy()
    lab = (t != -100).numpy()
    lse[~lab] = np.nan
    N = int(lab.sum())
    g = si.make_grad_output(t, red, c["seed"], scalar=1.0) if red == "none" else None
    print(f"[{cid}] BT={BT} H={H} V={V} {dt} chunk={chunk} {red} "
          f"share={share} seq={seq} frozen={frozen}", flush=True)

    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), reduction=red, chunk_size=chunk or None,
        accum_dtype=torch.float32 if accum == "f32" else None, frozen_weight=frozen,
        grad_output=None if g is None else g.to(dev), return_row_index=True)
    torch.cuda.synchronize()

    # compaction: the index list itself, bit for bit
    idx_ref, n_ref = oracle.compact(t, V)
    assert r.stats["n_valid"] == N == n_ref
    got_idx = r.row_index.cpu().numpy()
    assert got_idx.dtype == np.int32 and got_idx.shape == (N,)
    np.testing.assert_array_equal(got_idx.astype(np.int64), idx_ref)

    # ignored rows: exact +0.0 everywhere (no sign bit)
    ign_t = torch.from_numpy(np.nonzero(~lab)[0]).to(dev)
    if ign_t.numel():
        bits = r.dX[ign_t].view(torch.int16 if dt != "f32" else torch.int32)
        assert int(bits.abs().max()) == 0

    # loss
    zt = oracle.target_logits(Xd, Wd, t)
    ref_loss = oracle.loss_from_lse(lse, zt, t, reduction=red)
    if red == "none":
        got = r.loss.cpu().numpy()
        assert np.all(got[~lab] == 0.0) and not np.signbit(got[~lab]).any()
        loss_err = _rel(got[lab], ref_loss[lab])
    else:
        loss_err = abs(float(r.loss) - ref_loss) / abs(ref_loss)
    assert loss_err <= tl, loss_err

    # sampled grad_input rows
    rng = np.random.Generator(np.random.PCG64(7))
    csz = r.stats["chunk_size"]
    rows = _dx_picks(np.nonzero(lab)[0], csz, rng)
    dx_ref, lrow, _ = oracle.dx_rows_matmul(Xd, Wd, t, rows, n_valid=N, reduction=red,
                                            grad_output=g)
    dx_got = r.dX[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
    dx_err = _rel(dx_got, dx_ref)
    dx_rows_err = _row_errors(dx_got, dx_ref)
    worst = int(np.argmax(dx_rows_err))
    assert dx_err <= tg, dx_err
    assert dx_rows_err.max() <= tg, (int(rows[worst]), float(dx_rows_err[worst]))
    if red == "none":
        got_l = r.loss.cpu().numpy()[rows]
        assert float(np.max(np.abs(got_l - lrow) / np.abs(lrow))) <= tl

    # sampled grad_weight rows
    if not frozen:
        splits = r.stats["dx_splits"]
        ldz = -(-V // 8) * 8
        kps = -(-(-(-ldz // splits)) // 64) * 64  # the split width over V, as the library sets it
        bounds = [k * kps for k in range(1, splits)]
        vrows = _dw_picks(V, bounds, t.numpy()[rows[:8]], rng)
        dw_ref = oracle.dw_rows_matmul(Xd, Wd, t, vrows, lse, n_valid=N, reduction=red,
                                       grad_output=g)
        dw_got = r.dW[torch.from_numpy(vrows).to(dev)].double().cpu().numpy()
        dw_err = _rel(dw_got, dw_ref)
        dw_rows_err = _row_errors(dw_got, dw_ref,
                                  _storage_floor(dt, accum, r.stats["chunks_run"]))
        worst = int(np.argmax(dw_rows_err))
        assert dw_err <= tg, dw_err
        assert dw_rows_err.max() <= tg, (int(vrows[worst]), float(dw_rows_err[worst]))
        colsum = r.dW.double().sum(0)
        scale = r.dW.double().abs().sum(0)
        assert float((colsum.abs() / scale.clamp_min(1e-30)).max()) <= 5e-2
    else:
        dw_err = float("nan")
        vrows = np.zeros(0)
    print(f"[{cid}] {rows.size} dX rows, {vrows.size} dW rows; rel errors: loss {loss_err:.2e}  "
          f"dX {dx_err:.2e} (worst row {dx_rows_err.max():.2e})  dW {dw_err:.2e}", flush=True)


@pytest.mark.parametrize("mask", ["scattered", "prompt_first", "packed", "none", "all"])
@pytest.mark.parametrize("ignore_index", [-100, 17])
def test_compaction_index_bit_exact(pkg, mask, ignore_index):
    """The int32 labelled-row index of a BT = 32768 call equals the oracle's
    compaction bit for bit, for scattered, prompt-first (one sequence),
    packed (32 sequences of 1024, each prompt-first) masks, none ignored and
    all ignored, with ignore_index outside and inside [0, V) (PR #1554,
    Summary: nonzero() of the not-ignored mask, ascending)."""
    BT, H, V = 32768, 64, 1000
    seed = 4242
    X = si.make_x(BT, H, "bf16", seed)
    W = si.make_w(V, H, "bf16", seed)
    if mask in ("scattered", "prompt_first"):
        t = si.make_targets(BT, V, seed, ignore=mask, frac=0.37, ignore_index=ignore_index)
    else:
        t = si.make_targets(BT, V, seed, ignore_index=ignore_index)
        if mask == "packed":
            for s0 in range(0, BT, 1024):
                t[s0:s0 + 300] = ignore_index
        elif mask == "all":
            t[:] = ignore_index
    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        X.to(dev), W.to(dev), t.to(dev), ignore_index=ignore_index, reduction="sum",
        chunk_size=4096, frozen_weight=True, return_row_index=True)
    torch.cuda.synchronize()
    idx_ref, n_ref = oracle.compact(t, V, ignore_index)
    assert r.stats["n_valid"] == n_ref
    assert r.stats["chunks_run"] == -(-n_ref // 4096)
    got = r.row_index.cpu().numpy()
    assert got.dtype == np.int32
    np.testing.assert_array_equal(got.astype(np.int64), idx_ref)
