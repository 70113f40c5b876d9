"""Seeded synthetic inputs for fused linear cross-entropy.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  The CPU oracle and the GPU path both read the arrays it
returns, so the two sides see identical stored values.

Recipe (one ``numpy.random.Generator(PCG64)`` sub-stream per tensor):
  X       ~ N(0, 1)        drawn in float32, cast once to the operand dtype (RNE)
  W       ~ N(0, 0.02^2)   drawn in float32, cast once to the operand dtype (RNE)
  targets ~ uniform integers in [0, V)
  ignored rows (set to ignore_index):
    "scattered"    round(frac * BT) rows picked by a seeded permutation
    "prompt_first" in each sequence of ``seq_len`` rows, the first
                   round((1 - share) * seq_len) rows, as in the masked-SFT
                   benchmark of PR #1554 (labels: the first (1 - share) of each
                   sequence is ignored)
  grad_output: mean/sum -> one float32 scalar (1.0 unless asked otherwise);
               none     -> float32 U[0.5, 1.5) per row, NaN at ignored rows
Sub-stream seeds are seed+0 (X), +1 (W), +2 (targets), +3 (mask), +4 (grad_output).
"""
from __future__ import annotations

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(seed: int, shape, scale: float, dtype: torch.dtype) -> torch.Tensor:
    a = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return torch.from_numpy(a).to(dtype)


def make_x(BT: int, H: int, dtype: str, seed: int) -> torch.Tensor:
    return _normal(seed + 0, (BT, H), 1.0, DTYPES[dtype])


def make_w(V: int, H: int, dtype: str, seed: int, scale: float = 0.02) -> torch.Tensor:
    return _normal(seed + 1, (V, H), scale, DTYPES[dtype])


def make_targets(BT: int, V: int, seed: int, *, ignore: str = "none", frac: float = 0.0,
                 seq_len: int | None = None, ignore_index: int = -100) -> torch.Tensor:
    """Targets in [0, V); ``frac`` is the IGNORED share of rows."""
    t = _rng(seed + 2).integers(0, V, size=BT, dtype=np.int64)
    if ignore == "scattered":
        n_ign = int(round(frac * BT))
        perm = _rng(seed + 3).permutation(BT)
        t[perm[:n_ign]] = ignore_index
    elif ignore == "prompt_first":
        L = seq_len or max(BT, 1)
        for s0 in range(0, BT, L):
            n = min(L, BT - s0)
            t[s0:s0 + int(round(frac * n))] = ignore_index
    elif ignore == "all":
        t[:] = ignore_index
    elif ignore != "none":
        raise ValueError(f"unknown ignore pattern {ignore!r}")
    return torch.from_numpy(t)


def make_grad_output(targets: torch.Tensor, reduction: str, seed: int, *,
                     scalar: float = 1.0, ignore_index: int = -100,
                     nan_at_ignored: bool = True) -> torch.Tensor:
    if reduction in ("mean", "sum"):
        return torch.tensor([scalar], dtype=torch.float32)
    g = _rng(seed + 4).uniform(0.5, 1.5, size=targets.numel()).astype(np.float32)
    if nan_at_ignored:
        g[targets.numpy() == ignore_index] = np.nan
    return torch.from_numpy(g)


def make_case(BT: int, H: int, V: int, dtype: str, seed: int, **target_kw):
    """X, W, targets for one seeded case (CPU tensors)."""
    return (make_x(BT, H, dtype, seed), make_w(V, H, dtype, seed),
            make_targets(BT, V, seed, **target_kw))


# The five workloads, by what they are.  ``seed`` is 1000 + position.
WORKLOADS = {
    "tiny": dict(BT=256, H=128, V=1024, dtype="f32", chunk_size=64, ignore="scattered",
                 frac=0.10, reduction="mean", accum="f32", seed=1000),
    "llama3_8b_lm_head": dict(BT=8192, H=4096, V=128256, dtype="bf16", chunk_sizes=(256, 2048),
                              ignore="none", frac=0.0, reduction="mean", accum="f32", seed=1001),
    "same_dtype_sweep": dict(BT=16384, H=4096, V=32000, dtypes=("bf16", "f16", "f32"),
                             ignore="none", frac=0.0, reduction="mean", accum="same", seed=1002),
    "long_seq_large_vocab": dict(BTs=(8192, 32768), H=5376, V=262144, dtype="bf16",
                                 chunk_sizes=(0, 256), ignore="none", frac=0.0,
                                 reduction="mean", accum="same", seed=1003),
    "masked_sft": dict(BT=8192, H=2048, V=151936, dtype="bf16", labelled=(1.0, 0.75, 0.5, 0.1),
                       ignore="prompt_first", reductions=("sum", "none"), accum="same",
                       seed=1004),
}
