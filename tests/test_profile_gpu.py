"""Live per-kernel timing through the C ABI: a full profile counts every kernel
the call enqueues, and a profile limited to some kinds counts exactly those,
with the same launch counts.  The results of the call do not depend on
whether or what is profiled."""
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


def _call(pkg, dev, BT=700, H=256, V=1500, chunk=256):
    X, W, t = si.make_case(BT, H, V, "bf16", 4242, ignore="scattered", frac=0.25)
    Xd, Wd, td = X.to(dev), W.to(dev), t.to(dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    dX = torch.empty_like(Xd)
    dW = torch.empty(V, H, dtype=torch.float32, device=dev)
    wsb = pkg.flce_workspace_bytes(BT, H, V, pkg.BF16, chunk, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = pkg.FlceStats()

    def run():
        rc = pkg.flce_fwd_bwd(Xd.data_ptr(), Wd.data_ptr(), td.data_ptr(), BT, H, V, pkg.BF16,
                              -100, pkg.MEAN, chunk, 1, pkg.F32, 0, 0, None, loss.data_ptr(),
                              dX.data_ptr(), dW.data_ptr(), ws.data_ptr(), wsb,
                              torch.cuda.current_stream(dev).cuda_stream, st)
        torch.cuda.synchronize()
        assert rc == 0, pkg.flce_status_string(rc)
        return loss.clone(), dX.clone(), dW.clone()
    return run, st


def test_profile_kind_mask(pkg):
    dev = torch.device("cuda:0")
    run, st = _call(pkg, dev)
    ref = run()  # unprofiled
    assert pkg.flce_profile_begin() == 0
    full_out = run()
    full = pkg.flce_profile_end()
    n = st.chunks_run
    assert n == -(-st.n_valid // st.chunk_size) and n >= 2
    for k in ("logits_gemm", "softmax_grad", "dx_gemm", "dw_gemm", "gather_rows"):
        assert full[k][0] == n and full[k][1] > 0.0, k
    assert full["mask_scan"][0] == 1 and full["loss_finalize"][0] == 1

    assert pkg.flce_profile_begin_kinds(["dw_gemm", "logits_gemm"]) == 0
    part_out = run()
    part = pkg.flce_profile_end()
    assert part["dw_gemm"][0] == n and part["logits_gemm"][0] == n
    assert all(v == (0, 0.0) for k, v in part.items() if k not in ("dw_gemm", "logits_gemm"))

    for a, b, c in zip(ref, full_out, part_out):
        assert torch.equal(a, b) and torch.equal(a, c)
