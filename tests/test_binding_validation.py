"""The Python binding refuses operands that do not hold what the kernels address.

The kernels size their buffer descriptors from (m, n, k, group), not from the
allocations, so a short tensor would be read or written out of bounds on the
device.  The binding therefore checks every size before any library call;
these checks run before the device check, so they are exercised here on CPU
tensors (a correctly sized call then stops at "x must be on the GPU").
"""
import pytest
import torch

import weight_only_quantization_amd as woq

M, N, K, G = 2, 48, 256, 64
NG = K // G


@pytest.fixture(scope="module", autouse=True)
def _lib():
    woq.load()


def _ops(**over):
    ops = dict(
        x=torch.zeros((M, K), dtype=torch.bfloat16),
        packed=torch.zeros((N, K // 2), dtype=torch.uint8),
        scale=torch.ones((N, NG), dtype=torch.float32),
        zero=torch.zeros((N, NG), dtype=torch.uint8),
        bias=None, order=None, out=None,
    )
    ops.update(over)
    return ops


def _linear(**over):
    o = _ops(**over)
    return woq.linear_int4_groups(o["x"], o["packed"], o["scale"], o["zero"], bias=o["bias"], order=o["order"],
                                  group=G, out=o["out"], out_dtype=torch.float32)


def test_correct_sizes_reach_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        _linear(bias=torch.zeros(N), order=torch.arange(K, dtype=torch.int32),
                out=torch.empty((M, N), dtype=torch.float32))


@pytest.mark.parametrize("name,bad", [
    ("out", torch.empty((M, N + 1), dtype=torch.float32)),
    ("out", torch.empty((M + 1, N), dtype=torch.float32)),
    ("bias", torch.zeros(N - 1)),
    ("order", torch.arange(K - 1, dtype=torch.int32)),
    ("zero", torch.zeros((N, NG - 1), dtype=torch.uint8)),
    ("zero", torch.zeros((N - 1, NG), dtype=torch.uint8)),
])
def test_linear_rejects_missized_operands(name, bad):
    with pytest.raises(ValueError, match=name):
        _linear(**{name: bad})


def test_linear_rejects_scale_of_another_group_count():
    # scale [N, 3] with an explicit group of 64 (K / 64 = 4 groups)
    with pytest.raises(ValueError, match="scale"):
        _linear(scale=torch.ones((N, 3), dtype=torch.float32))


def test_linear_rejects_x_of_another_k():
    with pytest.raises(ValueError, match="inputs"):
        _linear(x=torch.zeros((M, K + 64), dtype=torch.bfloat16))


def test_prepared_rejects_short_buffer():
    with pytest.raises(ValueError, match="prepared"):
        woq.linear_int4_groups_prepared(torch.zeros((M, K), dtype=torch.bfloat16),
                                        torch.zeros(woq.prepared_bytes(N, K) - 16, dtype=torch.uint8),
                                        torch.ones((N, NG)), torch.zeros((N, NG), dtype=torch.uint8))


def test_zp4_rejects_missized_operands():
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    p = torch.zeros((N, K // 2), dtype=torch.uint8)
    s = torch.ones((N, NG))
    zp = torch.zeros((N, (NG + 1) // 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="zero_packed"):
        woq.linear_int4_groups_zp4(x, p, s, zp[:, :1].contiguous(), group=G)
    with pytest.raises(ValueError, match="bias"):
        woq.linear_int4_groups_zp4(x, p, s, zp, bias=torch.zeros(N + 1), group=G)
    with pytest.raises(ValueError, match="out"):
        woq.linear_int4_groups_zp4(x, p, s, zp, group=G, out=torch.empty((M, N - 1), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="on the GPU"):
        woq.linear_int4_groups_zp4(x, p, s, zp, group=G)


def test_grouped_rejects_missized_operands():
    x = torch.zeros((M, K), dtype=torch.bfloat16)

    def mat(n, zero_groups=NG, bias=None):
        return (torch.zeros((n, K // 2), dtype=torch.uint8), torch.ones((n, NG)),
                torch.zeros((n, zero_groups), dtype=torch.uint8), bias)

    with pytest.raises(ValueError, match="zero"):
        woq.linear_int4_groups_grouped(x, [mat(16), mat(32, zero_groups=NG - 1)])
    with pytest.raises(ValueError, match="bias"):
        woq.linear_int4_groups_grouped(x, [mat(16, bias=torch.zeros(15))])
    with pytest.raises(ValueError, match="out"):
        woq.linear_int4_groups_grouped(x, [mat(16), mat(32)],
                                       outs=[torch.empty((M, 16), dtype=torch.bfloat16),
                                             torch.empty((M, 31), dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="one output per matrix"):
        woq.linear_int4_groups_grouped(x, [mat(16), mat(32)], outs=[torch.empty((M, 16), dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="on the GPU"):
        woq.linear_int4_groups_grouped(x, [mat(16), mat(32)])


def test_sym_mxfp4_rows_reject_missized_operands():
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    p = torch.zeros((N, K // 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="bias"):
        woq.linear_int4_sym(x, p, torch.ones((N, K // 32), dtype=torch.float16), bias=torch.zeros(N + 2))
    with pytest.raises(ValueError, match="order"):
        woq.linear_int4_sym(x, p, torch.ones((N, K // 32), dtype=torch.float16),
                            order=torch.arange(K + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="bias"):
        woq.linear_mxfp4(x, p, torch.zeros((N, K // 32), dtype=torch.uint8), bias=torch.zeros(3))
    with pytest.raises(ValueError, match="out"):
        woq.linear_mxfp4(x, p, torch.zeros((N, K // 32), dtype=torch.uint8),
                         out=torch.empty((N, M), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="order"):
        woq.linear_int4_rows(x, p, torch.ones(N), order=torch.arange(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="on the GPU"):
        woq.linear_int4_rows(x, p, torch.ones(N))
