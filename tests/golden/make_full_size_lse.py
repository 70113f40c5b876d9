"""Write the stored expected values for the full-size parity tests.

For each full-size workload this computes, with the fp64 oracle only, the
log-sum-exp of every row's logits (lse_i = log sum_v exp(X_i . W_v)) on the
seeded synthetic inputs of that workload, and saves it with a fingerprint of
the inputs.  The GPU tests derive the mean/sum loss, sampled grad_input rows
and sampled grad_weight rows from it with the oracle's row functions, which
are cheap once lse is known.  Rows are treated as labelled here; a test
masks whatever its workload ignores.

Usage:  python tests/golden/make_full_size_lse.py [OUT_DIR] [NAME ...]
(default OUT_DIR: tests/golden/full_size).  The lse uses the oracle's
matmul variant (numpy fp64 matrix products), pinned to the loop oracle by
tests/test_oracle_pins.py.
"""
import hashlib
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402

# name: (BT, H, V, dtype, seed) -- the inputs of the benchmark workloads
SETS = {
    "llama3_8b_lm_head": (8192, 4096, 128256, "bf16", 1001),
    "same_dtype_sweep_bf16": (16384, 4096, 32000, "bf16", 1002),
    "same_dtype_sweep_f16": (16384, 4096, 32000, "f16", 1002),
    "same_dtype_sweep_f32": (16384, 4096, 32000, "f32", 1002),
    "long_seq_large_vocab": (32768, 5376, 262144, "bf16", 1003),
    "masked_sft": (8192, 2048, 151936, "bf16", 1004),
}


def fingerprint(X, W, t) -> str:
    h = hashlib.sha256()
    for a in (X.view(-1)[:4096], X.view(-1)[-4096:], W.view(-1)[:4096], W.view(-1)[-4096:]):
        h.update(a.float().numpy().tobytes())
    h.update(t.numpy().tobytes())
    return h.hexdigest()[:16]


def main():
    out = sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "tests", "golden", "full_size")
    names = sys.argv[2:] or list(SETS)
    os.makedirs(out, exist_ok=True)
    for name in names:
        BT, H, V, dt, seed = SETS[name]
        t0 = time.time()
        X = si.make_x(BT, H, dt, seed)
        W = si.make_w(V, H, dt, seed)
        t = si.make_targets(BT, V, seed)
        Xd, Wd = oracle.widen(X), oracle.widen(W)
        lse = oracle.lse_matmul(Xd, Wd, t, rows_per_block=256)
        np.savez(os.path.join(out, f"{name}.npz"), lse=lse, BT=BT, H=H, V=V, dtype=dt, seed=seed,
                 fingerprint=fingerprint(X, W, t))
        print(f"{name}: BT={BT} H={H} V={V} {dt} lse mean {np.mean(lse):.6f} "
              f"({time.time() - t0:.1f} s)", flush=True)
        del X, W, Xd, Wd


if __name__ == "__main__":
    main()
