"""GPU Int4Linear (signed int4, one float32 scale a row) against the float64 oracle.

linnet "Quantization", std.quant table (Int4Linear, dequantize_int4) with the
quantizer of tinyllm L8.5 section 2 at q_max = 7: the quantizer and
dequantization bit for bit, the linear layer on every path to the same bar as
the group layouts.  Each case prints its name first.
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


@pytest.mark.parametrize("n,k,std", [(64, 256, 0.02), (37, 96, 3.0), (5, 4100, 1e-3), (300, 2, 0.5)])
def test_quantize_matches_oracle(woq, n, k, std):
    _say(f"rows quantize n={n} k={k} std={std}")
    w = (np.random.default_rng(n + k).standard_normal((n, k)) * std).astype(np.float32)
    w[0] = 0.0
    if n > 1 and k >= 4:
        w[1] = 0.0                           # amax 0.4375 -> s = 0.0625: a tie at 3.5 steps (to 4), and -2
        w[1, :3] = [0.4375, 0.21875, -0.125]
    c, s = woq.quantize_int4_rows(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.quantize_int4_rows(w)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(c.cpu().numpy(), c_ref)


def test_quantize_refuses_nonfinite(woq):
    _say("rows quantize errors")
    bad = torch.zeros((3, 64), dtype=torch.float32, device="cuda")
    bad[2, 5] = float("nan")
    with pytest.raises(woq_mod.WoqError) as e:
        woq.quantize_int4_rows(bad)
    assert e.value.status == 4


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bit_exact(woq, out):
    _say(f"rows dequantize {out}")
    w = workloads.weight(33, 192, seed=5)
    c, s = woq.quantize_int4_rows(torch.from_numpy(w).cuda())
    packed = woq.pack_int4(c)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    got = woq.dequantize_int4_rows(packed, s, out_dtype=dt)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.quantize_int4_rows(w)
    want = oracle.dequantize_int4_rows(oracle.pack_int4(c_ref), s_ref, 33, 192, out=out)
    g = got.cpu()
    g = g.numpy() if out == "f32" else g.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(g, want)


def _make(woq, m, n, k, seed, with_bias, with_order):
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 2)
    b = workloads.bias(n, seed=seed + 3) if with_bias else None
    o = workloads.order(k, seed=seed + 4) if with_order else None
    c, s = woq.quantize_int4_rows(torch.from_numpy(w).cuda())
    dev = dict(x=to_dev_bf16(x), packed=woq.pack_int4(c), scale=s,
               bias=None if b is None else torch.from_numpy(b).cuda(),
               order=None if o is None else torch.from_numpy(o).cuda())
    return dev, dict(w=w, x=x, b=b, o=o)


def _ref(host, rows=None):
    w = host["w"] if rows is None else host["w"][rows]
    c, s = oracle.quantize_int4_rows(w)
    b = host["b"]
    if b is not None and rows is not None:
        b = b[rows]
    return oracle.linear_int4_rows(host["x"], oracle.pack_int4(c), s, w.shape[0], w.shape[1], bias=b,
                                   order=host["o"])


SMALL = [
    # m, n, k, bias, order; k picks the kernels' group (the largest of 256..32 dividing it)
    (1, 64, 256, False, False),
    (1, 100, 96, True, False),
    (2, 48, 4096, False, True),
    (4, 256, 640, True, False),
    (9, 31, 352, False, True),
    (32, 300, 1024, True, False),
    (33, 257, 1024, True, False),
    (130, 300, 384, True, True),
]


@pytest.mark.parametrize("m,n,k,with_bias,with_order", SMALL)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_small(woq, m, n, k, with_bias, with_order, out):
    _say(f"rows linear m={m} n={n} k={k} bias={with_bias} order={with_order} {out}")
    dev, host = _make(woq, m, n, k, seed=5 * m + n, with_bias=with_bias, with_order=with_order)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = woq.linear_int4_rows(dev["x"], dev["packed"], dev["scale"], bias=dev["bias"], order=dev["order"],
                             out_dtype=dt)
    torch.cuda.synchronize()
    check_linear(y, _ref(host), f"rows m={m} n={n} k={k}")


@pytest.mark.slow
@pytest.mark.parametrize("m,n,k", [(1, 14336, 4096), (2048, 4096, 4096)])
def test_full_size_sampled(woq, m, n, k):
    _say(f"rows full size m={m} n={n} k={k}")
    dev, host = _make(woq, m, n, k, seed=180 + m, with_bias=True, with_order=False)
    y = woq.linear_int4_rows(dev["x"], dev["packed"], dev["scale"], bias=dev["bias"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    rng = np.random.default_rng(n + 2)
    rows = np.unique(np.concatenate([[0, n - 1, n // 2], rng.choice(n, 48, replace=False)]))
    check_linear(y[:, torch.from_numpy(rows).cuda()], _ref(host, rows), f"rows full m={m}")
