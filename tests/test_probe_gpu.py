"""The benchmark's measurement probes (include/flce_probe.h) compute what they
claim, so that the ceilings `bench.py` reports measure real work.

* the read stream visits every 16-byte element once: the XOR of all threads'
  sinks equals the XOR of the whole buffer (checked on the host);
* each MFMA loop (32x32x16 and 16x16x32) with all-zero operands leaves zero in
  every sink, and with iters = 0 too; with random operands the sums are finite.
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
