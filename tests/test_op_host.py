"""The torch custom ops' schemas and fake (shape-only) implementations, on the
CPU: what torch.compile sees when it traces a call without running it."""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode


@pytest.fixture(scope="module")
def ops(flce_lib):
    return torch.ops.flce


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("accum_fp32", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_forward_fake_shapes(ops, reduction, accum_fp32, with_bias):
    with FakeTensorMode():
        x = torch.empty(10, 16, dtype=torch.bfloat16)
        w = torch.empty(33, 16, dtype=torch.bfloat16)
        t = torch.empty(10, dtype=torch.int64)
        b = torch.empty(33, dtype=torch.bfloat16) if with_bias else None
        loss, dx, dw, db = ops.fused_linear_cross_entropy(x, w, t, b, -100, reduction, 0, 1,
                                                          accum_fp32, False, 0.0, True)
        assert loss.shape == ((10,) if reduction == "none" else ()) and loss.dtype == torch.float32
        adt = torch.float32 if accum_fp32 else torch.bfloat16
        if reduction == "none":  # loss only; backward re-enters
            assert dx.numel() == 0 and dw.numel() == 0 and db.numel() == 0
        else:
            assert dx.shape == x.shape and dx.dtype == x.dtype
            assert dw.shape == w.shape and dw.dtype == adt
            assert (db.shape == (33,) and db.dtype == adt) if with_bias else db.numel() == 0


def test_backward_fake_shapes(ops):
    with FakeTensorMode():
        x = torch.empty(7, 8, dtype=torch.float16)
        w = torch.empty(20, 8, dtype=torch.float16)
        t = torch.empty(7, dtype=torch.int64)
        g = torch.empty(7, dtype=torch.float32)
        dx, dw, db = ops.fused_linear_cross_entropy_backward(x, w, t, None, g, -100, "none", 0, 1,
                                                             True, False, 0.0)
        assert dx.shape == x.shape and dw.shape == w.shape and dw.dtype == torch.float32
        assert db.numel() == 0


def test_frozen_weight_has_no_weight_gradient(ops):
    with FakeTensorMode():
        x = torch.empty(4, 8, dtype=torch.bfloat16)
        w = torch.empty(12, 8, dtype=torch.bfloat16)
        t = torch.empty(4, dtype=torch.int64)
        _, dx, dw, _ = ops.fused_linear_cross_entropy(x, w, t, None, -100, "mean", 0, 1, False,
                                                      True, 0.0, True)
        assert dx.shape == x.shape and dw.numel() == 0
