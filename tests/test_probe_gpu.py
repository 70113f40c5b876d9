"""The benchmark's measurement probes (include/flce_probe.h) compute what they
claim, so that the ceilings `bench.py` reports measure real work.

* the read stream visits every 16-byte element once: the XOR of all threads'
  sinks equals the XOR of the whole buffer (checked on the host);
* each MFMA loop (32x32x16 and 16x16x32) with all-zero operands leaves zero in
  every sink, and with iters = 0 too; with random operands the sums are finite;
* with random operands each thread's sink matches a CPU model of the loop (its
  fragments, operand rotation and the MFMA lane layouts), so every MFMA the
  ceiling counts is executed.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "linear_cross_entropy_chunked_amd")


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(os.path.join(PKG, "libflce_probe.so"))
    for f in (lib.flce_probe_mfma_loop, lib.flce_probe_mfma16_loop):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.flce_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096 + 16, 3), (3 << 20, 7), (8 << 20, 8)])
def test_read_stream_visits_every_element(probe, nbytes, blocks):
    print(f"read stream: {nbytes} B over {blocks} workgroups", flush=True)
    g = torch.Generator().manual_seed(nbytes + blocks)
    host = torch.randint(0, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    dev = torch.device("cuda:0")
    src = host.to(dev)
    thr = probe.flce_probe_stream_threads()
    sink = torch.zeros(blocks * thr * 4, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    assert probe.flce_probe_read_stream(src.data_ptr(), nbytes, sink.data_ptr(),
                                        sink.numel() * 4, blocks, st) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().reshape(-1, 4), axis=0)
    want = np.bitwise_xor.reduce(host.numpy().reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("loop_name", ["flce_probe_mfma_loop", "flce_probe_mfma16_loop"])
def test_mfma_loop_zero_operands_and_no_iterations(probe, loop_name):
    print(f"{loop_name}: 4 workgroups", flush=True)
    loop = getattr(probe, loop_name)
    dev = torch.device("cuda:0")
    thr = probe.flce_probe_mfma_threads()
    blocks = 4
    st = torch.cuda.current_stream(dev).cuda_stream
    ops = torch.zeros(1 << 16, dtype=torch.bfloat16, device=dev)
    sink = torch.full((blocks * thr,), 7.0, device=dev)
    assert loop(ops.data_ptr(), ops.numel() * 2, sink.data_ptr(),
                sink.numel(), blocks, 50, st) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0
    rnd = (torch.randn(1 << 16, generator=torch.Generator().manual_seed(3)) * 0.05).to(
        torch.bfloat16).to(dev)
    sink.fill_(7.0)
    assert loop(rnd.data_ptr(), rnd.numel() * 2, sink.data_ptr(),
                sink.numel(), blocks, 0, st) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0
    assert loop(rnd.data_ptr(), rnd.numel() * 2, sink.data_ptr(),
                sink.numel(), blocks, 20, st) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all() and torch.count_nonzero(sink).item() > 0


def _mfma_loop_model(ops, threads, iters, sub16):
    """CPU model of the probe's MFMA loop for one workgroup: each lane's
    fragments, the operand rotation, and the MFMA lane layouts
    (32x32x16: lane l holds A[l % 32][8 (l / 32) + 0..7] and B[k][l % 32] for the
    same k; 16x16x32: A[l % 16][8 (l / 16) + 0..7] and B[k][l % 16]).  Returns
    each thread's sum over its accumulators (fp64; the products of bf16 values
    are exact)."""
    nops = ops.shape[0]
    sink = np.zeros(threads)
    n = 16 if sub16 else 32          # output block is n x n
    kg = 64 // n                     # lane groups along k
    nacc = 16 if sub16 else 8
    for w in range(threads // 64):
        lanes = np.arange(64) + 64 * w
        a = [ops[(lanes * 8 + i) % nops] for i in range(4)]        # each [64, 8]
        b = [ops[(lanes * 8 + 4 + i) % nops] for i in range(4)]
        acc = np.zeros((nacc, n, n))
        for _ in range(iters):
            for s in range(4):
                for j in range(nacc):
                    fa, fb = a[(s + j) & 3], b[(s + 3 * j) & 3]
                    A = np.zeros((n, 8 * kg)); B = np.zeros((8 * kg, n))
                    for l in range(64):
                        A[l % n, 8 * (l // n):8 * (l // n) + 8] = fa[l]
                        B[8 * (l // n):8 * (l // n) + 8, l % n] = fb[l]
                    acc[j] += A @ B
            x = a[0]
            a = [a[1], a[2], a[3], b[0]]
            b = [b[1], b[2], b[3], x]
        # per-lane ownership of the accumulator elements
        for l in range(64):
            if sub16:
                rows = [4 * (l // 16) + e for e in range(4)]
                sink[64 * w + l] = sum(acc[j][r, l % 16] for j in range(nacc) for r in rows)
            else:
                rows = [8 * (r >> 2) + 4 * (l >> 5) + (r & 3) for r in range(16)]
                sink[64 * w + l] = sum(acc[j][r, l % 32] for j in range(nacc) for r in rows)
    return sink


@pytest.mark.parametrize("loop_name,sub16", [("flce_probe_mfma_loop", False),
                                             ("flce_probe_mfma16_loop", True)])
def test_mfma_loop_matches_a_cpu_model(probe, loop_name, sub16):
    """Every MFMA of the loop runs on the operands the header describes: each
    thread's sink after two iterations matches the model to fp32 rounding."""
    print(f"{loop_name}: one workgroup, 2 iterations", flush=True)
    loop = getattr(probe, loop_name)
    dev = torch.device("cuda:0")
    thr = probe.flce_probe_mfma_threads()
    g = torch.Generator().manual_seed(11 + sub16)
    host = (torch.randn(thr * 8 * 8, generator=g) * 0.05).to(torch.bfloat16)
    ops = host.to(dev)
    sink = torch.full((thr,), 7.0, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    assert loop(ops.data_ptr(), ops.numel() * 2, sink.data_ptr(), sink.numel(), 1, 2, st) == 0
    torch.cuda.synchronize()
    ref = _mfma_loop_model(host.float().numpy().astype(np.float64).reshape(-1, 8), thr, 2, sub16)
    got = sink.cpu().numpy().astype(np.float64)
    scale = np.abs(ref).max()
    assert scale > 0
    assert np.abs(got - ref).max() <= 1e-4 * scale, np.abs(got - ref).max() / scale
