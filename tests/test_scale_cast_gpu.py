"""The library's scale/cast kernel (the wrapper tail: fp32 dW to the weight
dtype, and the upstream gradient scale) against torch's own conversion.

Every pair of the three dtypes, with and without a scale, at lengths that leave
0-7 elements after the 8-element vector body, at aligned and 2-byte-misaligned
addresses (the element-wise path): scale * x is rounded once, to nearest even,
exactly as torch's float -> half / bfloat16 conversion does, so the results
must agree bit for bit.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

DT = [torch.float32, torch.float16, torch.bfloat16]


@pytest.fixture(scope="module")
def pkg(flce_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return flce_lib


@pytest.mark.parametrize("src_dt", DT, ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("dst_dt", DT, ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000, 4099])
@pytest.mark.parametrize("scaled", [False, True])
@pytest.mark.parametrize("offset", [0, 1])
def test_scale_cast_matches_torch(pkg, src_dt, dst_dt, n, scaled, offset):
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(n + 7 * offset)
    base = (torch.randn(n + offset, generator=gen) * 3.0).to(src_dt).to(dev)
    src = base[offset:]
    scale = torch.tensor([0.37], device=dev) if scaled else None
    out = torch.full((n + offset,), 7.0, dtype=dst_dt, device=dev)[offset:]
    got = pkg.scale_cast(src, dst_dt, scale=scale, out=out)
    torch.cuda.synchronize()
    ref = (src.float() * (0.37 if scaled else 1.0)).to(dst_dt)
    assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))
