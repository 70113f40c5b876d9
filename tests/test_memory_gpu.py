"""Device memory of a call (issue #1323: no per-chunk [V, H] temporary;
PR #1439, Summary: the logits slab is chunk_size x V x itemsize).

With the inputs and outputs allocated beforehand, the peak of torch's
allocator over "allocate the workspace, call, free it" is the workspace
itself, up to the allocator's rounding of a block (at most 2 MiB); the
library allocates no device memory of its own (the device's free memory is
the same before and after a call); the transient is flat in BT at a fixed chunk size except for
the 8 bytes per row of index and per-row loss; and it stays far below one
[V, H] fp32 buffer.
"""
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


def _transient(pkg, BT, H, V, chunk, dtype="bf16"):
    dev = torch.device("cuda:0")
    X, W, t = si.make_case(BT, H, V, dtype, 6100 + BT, ignore="scattered", frac=0.1)
    Xd, Wd, td = X.to(dev), W.to(dev), t.to(dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    dX = torch.empty_like(Xd)
    dW = torch.empty(V, H, dtype=torch.float32, device=dev)
    dt = {"bf16": pkg.BF16, "f32": pkg.F32}[dtype]
    wsb = pkg.flce_workspace_bytes(BT, H, V, dt, chunk, 1)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(ws):
        rc = pkg.flce_fwd_bwd(Xd.data_ptr(), Wd.data_ptr(), td.data_ptr(), BT, H, V, dt, -100,
                              pkg.MEAN, chunk, 1, pkg.F32, 0, 0, None, loss.data_ptr(),
                              dX.data_ptr(), dW.data_ptr(), ws.data_ptr(), wsb, stream, None)
        assert rc == 0, pkg.flce_status_string(rc)

    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    call(ws)  # first call: code objects load, pinned host word allocated
    torch.cuda.synchronize()
    del ws
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    call(ws)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info(dev)[0]
    peak = torch.cuda.max_memory_allocated(dev) - m0
    del ws
    return wsb, peak, free0, free1


def test_transient_is_the_workspace_and_flat_in_bt(pkg):
    H, V, chunk = 1024, 32000, 64
    w1, p1, f0, f1 = _transient(pkg, 512, H, V, chunk)
    w2, p2, g0, g1 = _transient(pkg, 2048, H, V, chunk)
    mib2 = 2 << 20
    for w, p in ((w1, p1), (w2, p2)):
        assert w <= p <= -(-w // mib2) * mib2, (w, p)
    # flat in BT: only the int32 row index and the fp32 per-row loss grow with it
    assert w2 - w1 == 8 * (2048 - 512)
    # no [V, H] temporary: far below one fp32 dW
    assert p2 < V * H * 4 // 10
    # the slab dominates and is chunk x V x itemsize
    assert w1 >= chunk * V * 2


def test_library_allocates_no_device_memory(pkg):
    """The device's free memory does not change across a call whose workspace
    torch's allocator already holds (torch itself allocates nothing here)."""
    wsb, peak, free0, free1 = _transient(pkg, 1024, 512, 8192, 128)
    assert free1 >= free0, (free0, free1)
