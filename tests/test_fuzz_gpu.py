"""Seeded random configurations through the C ABI against the fp64 oracle.

Each case draws its own shape and options: operand dtype, BT (including 0
and 1), H (a multiple of 8), V (including 1 and sizes that are ragged against
every tile), chunk_size (heuristic with C = 1, 2, 8 or 16, the MI355X policy,
powers of two, values that floor to one),
dW in fp32 or the operand dtype, mean / sum / none, a frozen weight, dW
accumulation onto a random buffer, an ignored share from none to all rows
(scattered or prompt-first), an ignore_index inside [0, V) as well as -100,
and NaN planted in the ignored rows of X and of the per-token upstream
gradient.  The oracle sees the clean inputs; the HIP path must not notice the
NaN.  Tolerances as everywhere: fp32 loss 1e-5 and gradients 1e-4; 16-bit
loss 2e-3 and gradients 2e-2 (relative, Frobenius).  The labelled-row count
and every ignored-row output are exact.

A second generator draws larger shapes (BT 257-1499, H 192-512, V 1025-2999,
chunks of 256-1024 rows), which run the eight-wave 256 x 256 tiles of all three
GEMMs with ragged edges and several chunks per call.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2), "f16": (2e-3, 2e-2)}
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
N_CASES = 160


def draw(i):
    """The configuration of case i (a pure function of i)."""
    r = np.random.Generator(np.random.PCG64(90210 + i))
    pick = lambda xs: xs[int(r.integers(len(xs)))]
    dtype = pick(["f32", "bf16", "bf16", "f16"])
    BT = int(pick([0, 1, 7, int(r.integers(2, 130)), int(r.integers(130, 330)),
                   int(r.integers(130, 330)), int(r.integers(200, 600)), int(r.integers(200, 600))]))
    H = 8 * int(r.integers(1, 41))
    V = int(pick([1, 2, int(r.integers(3, 70)), int(r.integers(70, 700)),
                  int(r.integers(70, 700)), int(r.integers(700, 1500)),
                  int(r.integers(700, 1500))]))
    chunk = pick([None, None, 1, 3, 16, 64, 100, 128, 256, 512, 4096])
    accum = pick(["f32", "same"])
    reduction = pick(["mean", "sum", "none"])
    frozen = bool(r.random() < 0.15)
    accumulate = (not frozen) and bool(r.random() < 0.25)
    ignore = pick(["none", "scattered", "scattered", "scattered", "prompt_first",
                   "prompt_first", "all"])
    frac = float(pick([0.1, 0.5, 0.9]))
    ignore_index = -100 if r.random() < 0.7 else int(r.integers(0, V))
    poison = bool(r.random() < 0.5)
    scalar = float(pick([1.0, 0.5, 3.0]))
    # drawn last, so that the fields above keep their values: the heuristic's
    # memory multiplier C, and the MI355X policy in place of the heuristic
    policy = pick([None, None, "mi355x"])
    mem_const = int(pick([1, 1, 2, 8, 16]))
    if chunk is None and policy is not None:
        chunk = policy
    return dict(dtype=dtype, BT=BT, H=H, V=V, chunk=chunk, accum=accum, reduction=reduction,
                frozen=frozen, accumulate=accumulate, ignore=ignore, frac=frac,
                ignore_index=ignore_index, poison=poison, scalar=scalar, mem_const=mem_const,
                seed=5000 + 17 * i)


# cases 0-11 and four that accumulate into a given dW (16, 17, 22, 38)
LARGE_CASES = list(range(12)) + [16, 17, 22, 38]


def draw_large(i):
    """Case i of the larger shapes (a pure function of i)."""
    r = np.random.Generator(np.random.PCG64(777000 + i))
    pick = lambda xs: xs[int(r.integers(len(xs)))]
    dtype = pick(["f32", "bf16", "bf16", "f16"])
    BT = int(r.integers(257, 1500))
    H = 8 * int(r.integers(24, 65))
    V = int(r.integers(1025, 3000))
    chunk = pick([256, 300, 512, 640, 1024, None])
    return dict(dtype=dtype, BT=BT, H=H, V=V, chunk=chunk, accum=pick(["f32", "same"]),
                reduction=pick(["mean", "sum", "none"]), frozen=bool(r.random() < 0.1),
                accumulate=bool(r.random() < 0.3),
                ignore=pick(["none", "scattered", "prompt_first"]),
                frac=float(pick([0.1, 0.5])), ignore_index=-100, poison=bool(r.random() < 0.5),
                scalar=float(pick([1.0, 0.5])), mem_const=1, seed=70000 + 13 * i)


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
def test_random_configuration(pkg, i):
    _run_case(pkg, i, draw(i))


@pytest.mark.parametrize("i", LARGE_CASES)
def test_random_large_configuration(pkg, i):
    _run_case(pkg, i, draw_large(i))


def _run_case(pkg, i, c):
    dt, BT, H, V, ii = c["dtype"], c["BT"], c["H"], c["V"], c["ignore_index"]
    print(f"case {i}: {c}", flush=True)
    X = si.make_x(BT, H, dt, c["seed"])
    W = si.make_w(V, H, dt, c["seed"])
    t = si.make_targets(BT, V, c["seed"], ignore=c["ignore"], frac=c["frac"], ignore_index=ii)
    ign = (t == ii).numpy()
    g = si.make_grad_output(t, c["reduction"], c["seed"], scalar=c["scalar"], ignore_index=ii)
    adt = torch.float32 if c["accum"] == "f32" else TD[dt]
    dW0 = None
    if c["accumulate"]:
        dW0 = (torch.from_numpy(np.random.Generator(np.random.PCG64(c["seed"] + 9))
                                .standard_normal((V, H)).astype(np.float32)) * 0.01).to(adt)

    # GPU inputs: NaN in the ignored rows of X when poisoned (and always in the
    # per-token upstream gradient at ignored rows)
    Xg = X.clone()
    if c["poison"] and ign.any():
        Xg[torch.from_numpy(ign)] = float("nan")
    dev = torch.device("cuda:0")
    r = pkg.fused_linear_cross_entropy_fwd_bwd(
        Xg.to(dev), W.to(dev), t.to(dev), ignore_index=ii, reduction=c["reduction"],
        chunk_size=c["chunk"], chunk_mem_const=c["mem_const"],
        accum_dtype=adt if c["accum"] == "f32" else None,
        frozen_weight=c["frozen"], grad_output=g.to(dev),
        dW=None if dW0 is None else dW0.clone().to(dev), accumulate_dw=c["accumulate"])
    torch.cuda.synchronize()

    n_lab = int((~ign).sum())
    assert r.stats["n_valid"] == n_lab
    tl, tg = TOL[dt]
    dx = r.dX.float().cpu().numpy()
    assert np.all(dx[ign] == 0.0) and not np.signbit(dx[ign]).any()
    if not c["frozen"]:
        assert r.dW.dtype == adt

    if BT == 0 or n_lab == 0:
        # nothing labelled: zero loss, zero dX, dW untouched by any GEMM
        lo = r.loss.cpu().numpy()
        assert np.all(lo == 0.0)
        assert np.all(dx == 0.0)
        if not c["frozen"]:
            want = np.zeros((V, H)) if dW0 is None else dW0.double().numpy()
            assert np.array_equal(r.dW.double().cpu().numpy(), want)
        return

    if V == 1:
        # one class: every loss is exactly 0 and the exact gradients vanish.  The
        # fp32 path reproduces that exactly; 16-bit gradients carry the rounding of
        # the stored logits (bounded in test_parity_gpu.test_degenerate_shapes)
        assert np.all(r.loss.cpu().numpy() == 0.0)
        if dt == "f32":
            assert np.all(dx == 0.0)
            if not c["frozen"]:
                want = np.zeros((V, H)) if dW0 is None else dW0.double().numpy()
                assert np.array_equal(r.dW.double().cpu().numpy(), want)
        else:
            assert np.isfinite(dx).all()
        return

    gref = torch.nan_to_num(g)
    ref = oracle.flce(X, W, t, ignore_index=ii, reduction=c["reduction"], grad_output=gref,
                      frozen=c["frozen"], dW_init=dW0)
    assert ref["n_valid"] == n_lab
    if c["reduction"] == "none":
        lo = r.loss.cpu().numpy()
        assert np.all(lo[ign] == 0.0) and not np.signbit(lo[ign]).any()
        assert _rel(lo, ref["loss"]) <= tl
    else:
        lo = float(r.loss)
        assert abs(lo - ref["loss"]) <= tl * max(abs(ref["loss"]), 1e-30), (lo, ref["loss"])
    assert _rel(dx, ref["dX"]) <= tg, _rel(dx, ref["dX"])
    if not c["frozen"]:
        assert _rel(r.dW.double().cpu().numpy(), ref["dW"]) <= tg, \
            _rel(r.dW.double().cpu().numpy(), ref["dW"])
