"""GPU MXFP4 against the float64 oracle.

linnet "Quantization" (dequantize_mxfp4: E2M1 values in blocks of 32, one E8M0
scale byte a block) and tinyllm L8.5 section 2 ("MXFP4"): the quantizer and
dequantization bit for bit, the linear layer on the small-M and GEMM paths to
the same bar as the int4 layouts.  Each case prints its name first.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import weight_only_quantization_amd as woq_mod
from helpers import check_linear, to_dev_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _weights(n, k, seed, std=0.02):
    w = workloads.weight(n, k, seed=seed, std=std)
    if n > 2 and k >= 64:
        w[0, :32] = 0.0                       # a zero block
        w[1, 32:64] = 1e-41                   # a float32-subnormal block: scale byte 0
        w[2, 0:12] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.1, -0.3, 6.5, -0.0]
    return w


@pytest.mark.parametrize("n,k,std", [(64, 256, 0.02), (37, 96, 3.0), (16, 4096, 1e-4), (5, 32, 100.0)])
def test_quantize_matches_oracle(woq, n, k, std):
    _say(f"mxfp4 quantize n={n} k={k} std={std}")
    w = _weights(n, k, seed=n + k, std=std)
    c, e = woq.quantize_mxfp4(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    c_ref, e_ref = oracle.quantize_mxfp4(w)
    assert np.array_equal(e.cpu().numpy(), e_ref)
    assert np.array_equal(c.cpu().numpy(), c_ref)


def test_quantize_refuses_nonfinite(woq):
    _say("mxfp4 quantize errors")
    bad = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    bad[1, 40] = float("inf")
    with pytest.raises(woq_mod.WoqError) as e:
        woq.quantize_mxfp4(bad)
    assert e.value.status == 4


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_every_code_and_scale(woq, out):
    _say(f"mxfp4 dequantize all codes {out}")
    # every code at every E8M0 scale byte 0..254
    n, k = 255, 32
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, 2))
    scales = np.arange(255, dtype=np.uint8).reshape(n, 1)
    blocks = oracle.pack_uint4(codes)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    got = woq.dequantize_mxfp4(torch.from_numpy(blocks).cuda(), torch.from_numpy(scales).cuda(), out_dtype=dt)
    torch.cuda.synchronize()
    want = oracle.dequantize_mxfp4(blocks, scales, n, k, out=out)
    g = got.cpu()
    g = g.numpy() if out == "f32" else g.view(torch.int16).numpy().view(np.uint16)
    finite = np.isfinite(oracle.dequantize_mxfp4(blocks, scales, n, k))
    assert np.array_equal(g[finite], np.asarray(want)[finite])


def _make(woq, m, n, k, seed, with_bias):
    w = _weights(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 2)
    b = workloads.bias(n, seed=seed + 3) if with_bias else None
    c, e = woq.quantize_mxfp4(torch.from_numpy(w).cuda())
    dev = dict(x=to_dev_bf16(x), blocks=woq.pack_uint4(c), scales=e,
               bias=None if b is None else torch.from_numpy(b).cuda())
    return dev, dict(w=w, x=x, b=b)


def _ref(host, rows=None):
    w = host["w"] if rows is None else host["w"][rows]
    c, e = oracle.quantize_mxfp4(w)
    b = host["b"]
    if b is not None and rows is not None:
        b = b[rows]
    return oracle.linear_mxfp4(host["x"], oracle.pack_uint4(c), e, w.shape[0], w.shape[1], bias=b)


SMALL = [
    # m, n, k, bias (m <= 32: small-M kernel; above: tiled GEMM)
    (1, 64, 256, False),
    (1, 100, 96, True),
    (2, 48, 4096, False),
    (4, 256, 768, True),
    (5, 31, 352, False),
    (16, 512, 2048, True),
    (24, 1000, 1920, False),
    (32, 64, 160, False),
    (33, 257, 1024, True),
    (100, 300, 384, True),
    (256, 512, 1024, False),
    (200, 33064, 256, True),
]


@pytest.mark.parametrize("m,n,k,with_bias", SMALL)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_small(woq, m, n, k, with_bias, out):
    _say(f"mxfp4 linear m={m} n={n} k={k} bias={with_bias} {out}")
    dev, host = _make(woq, m, n, k, seed=3 * m + n, with_bias=with_bias)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = woq.linear_mxfp4(dev["x"], dev["blocks"], dev["scales"], bias=dev["bias"], out_dtype=dt)
    torch.cuda.synchronize()
    check_linear(y, _ref(host), f"mxfp4 m={m} n={n} k={k}")


FULL = [(1, 14336, 4096), (1, 4096, 14336), (16, 14336, 4096), (2048, 4096, 4096)]


@pytest.mark.slow
@pytest.mark.parametrize("m,n,k", FULL)
def test_full_size_sampled(woq, m, n, k):
    _say(f"mxfp4 full size m={m} n={n} k={k}")
    dev, host = _make(woq, m, n, k, seed=170 + m, with_bias=True)
    y = woq.linear_mxfp4(dev["x"], dev["blocks"], dev["scales"], bias=dev["bias"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    rng = np.random.default_rng(n + 1)
    rows = np.unique(np.concatenate([[0, n - 1, n // 2], rng.choice(n, 48, replace=False)]))
    check_linear(y[:, torch.from_numpy(rows).cuda()], _ref(host, rows), f"mxfp4 full m={m}")


# m <= 4: the row-streaming kernel (one E8M0 block per lane, converted with
# its scale) and the tile GEMV (WOQ_DECODE_MFMA; at k = 32768 with 32-input
# blocks it hands over to the small-M kernel) on the same calls.
DECODE = [(1, 300, 2048, True), (1, 37, 64, False), (2, 64, 4096, True), (3, 100, 6144, False),
          (4, 70, 1024, True), (1, 129, 32768, False)]


@pytest.mark.parametrize("kernel", ["rows", "gemv"])
@pytest.mark.parametrize("m,n,k,with_bias", DECODE)
def test_decode_paths(woq, monkeypatch, kernel, m, n, k, with_bias):
    if kernel == "gemv":
        monkeypatch.setenv("WOQ_DECODE_MFMA", "1")
    else:
        monkeypatch.delenv("WOQ_DECODE_MFMA", raising=False)
    plan = woq.linear_plan(m, n, k, 32)
    _say(f"mxfp4 decode {kernel} m={m} n={n} k={k} plan: {plan}")
    if kernel == "rows":
        assert "path=rows_dot2" in plan, plan
    else:   # the tile GEMV, or the small-M kernel for rows its LDS budget cannot take
        assert "path=gemv_mfma" in plan or (k >= 32768 and "path=skinny_mfma" in plan), plan
    dev, host = _make(woq, m, n, k, seed=7 * m + n + k, with_bias=with_bias)
    ref = _ref(host)
    for dt in (torch.float32, torch.bfloat16):
        y = woq.linear_mxfp4(dev["x"], dev["blocks"], dev["scales"], bias=dev["bias"], out_dtype=dt)
        torch.cuda.synchronize()
        check_linear(y, ref, f"mxfp4 decode {kernel} m={m} n={n} k={k}")
