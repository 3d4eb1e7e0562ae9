"""GPU small-M path with the activation slice in LDS against the float64 oracle.

linnet "Quantization", std.quant table (linear_int4_groups, dequantize then
linear).  From 5 to 64 activation rows a workgroup of 8 waves owns 8T weight
tiles of 16 rows and one K range of S 128-input steps; it loads the range's
activations into LDS once, and with more than one range each leaves a float32
partial that a second pass sums in range order.  Every launch shape
(T in {1, 2}, S in {4, 8}) runs on ragged rows, columns and K tails, with the
act-order gather, for every weight format: unsigned groups (byte and packed
zero points, canonical and prepared layouts), signed groups with float16
scales, Int4Linear rows and MXFP4.  Each case prints its name first.
"""
import sys

import pytest
import torch

import oracle
import workloads
from helpers import check_linear, to_dev_bf16

pytestmark = pytest.mark.gpu

CASES = [
    # m, n, k, group, bias, order
    (5, 100, 96, 32, False, False),       # one partial step (96 inputs), ragged n
    (16, 1000, 1920, 64, True, False),    # 15 steps: a partial last range
    (17, 300, 4160, 64, True, True),      # two activation tiles, a 64-input tail step
    (33, 257, 1024, 256, True, False),    # four activation tiles, 31 padding rows
    (64, 1000, 2048, 32, False, True),
    (48, 640, 8192, 128, True, False),
    (8, 4096, 4096, 128, False, True),
]
SHAPES = ["1,4", "2,4", "1,8", "2,8"]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _force(woq, monkeypatch, shape, m, n, k, group, has_order):
    """Force the LDS small-M path with launch shape `shape`; None if it does not fit."""
    monkeypatch.setenv("WOQ_SM", shape)
    plan = woq.linear_plan(m, n, k, group, has_order)
    fields = dict(f.split("=", 1) for f in plan.split())
    if fields["path"] != "smallm_lds":
        return None
    t, s = shape.split(",")
    assert fields["weight_tiles_per_wave"] == t and fields["steps_per_range"] == s, plan
    return plan


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("m,n,k,group,with_bias,with_order", CASES)
def test_groups(woq, monkeypatch, shape, m, n, k, group, with_bias, with_order):
    plan = _force(woq, monkeypatch, shape, m, n, k, group, with_order)
    if plan is None:
        pytest.skip(f"shape {shape} does not fit LDS at m={m} g={group}")
    _say(f"smallm groups m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} plan: {plan}")
    seed = 9900 + m + n + k
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    b = workloads.bias(n, seed=seed + 2) if with_bias else None
    o = workloads.order(k, seed=seed + 3) if with_order else None
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
    packed = woq.pack_uint4(q)
    qr, sr, zr = oracle.quantize_groups(w, group)
    ref = oracle.linear_int4_groups(x, oracle.pack_uint4(qr), sr, zr, n, k, group, bias=b, order=o)
    dev_b = None if b is None else torch.from_numpy(b).cuda()
    dev_o = None if o is None else torch.from_numpy(o).cuda()
    ys = {}
    for out in (torch.float32, torch.bfloat16):
        y = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z, bias=dev_b, order=dev_o, group=group,
                                   out_dtype=out)
        again = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z, bias=dev_b, order=dev_o, group=group,
                                       out_dtype=out)
        torch.cuda.synchronize()
        assert torch.equal(y, again), "the ranges are summed in a fixed order"
        check_linear(y, ref, f"smallm m={m} {shape} {out}")
        ys[out] = y
    # the prepared layout feeds the same kernel: bit-identical
    yp = woq.linear_int4_groups_prepared(to_dev_bf16(x), woq.prepare_int4(packed), s, z, bias=dev_b,
                                         order=dev_o, out_dtype=torch.float32)
    # packed zero points: bit-identical to the byte zero points
    yz = woq.linear_int4_groups_zp4(to_dev_bf16(x), packed, s, woq.pack_zero_points(z), bias=dev_b,
                                    order=dev_o, group=group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(yp, ys[torch.float32])
    assert torch.equal(yz, ys[torch.float32])


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("m,n,k,group,with_bias,with_order", CASES)
def test_signed_f16_scales(woq, monkeypatch, shape, m, n, k, group, with_bias, with_order):
    plan = _force(woq, monkeypatch, shape, m, n, k, group, with_order)
    if plan is None:
        pytest.skip(f"shape {shape} does not fit LDS at m={m} g={group}")
    _say(f"smallm sym16 m={m} n={n} k={k} g={group} plan: {plan}")
    seed = 9910 + m + n + k
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    b = workloads.bias(n, seed=seed + 2) if with_bias else None
    o = workloads.order(k, seed=seed + 3) if with_order else None
    c, s16 = woq.quantize_int4_sym(torch.from_numpy(w).cuda(), group)
    cr, sr = oracle.quantize_int4_sym_f16(w, group)
    ref = oracle.linear_int4_sym_f16(x, oracle.pack_int4(cr), sr, n, k, group, bias=b, order=o)
    y = woq.linear_int4_sym(to_dev_bf16(x), woq.pack_int4(c), s16,
                            bias=None if b is None else torch.from_numpy(b).cuda(),
                            order=None if o is None else torch.from_numpy(o).cuda(), group=group,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_linear(y, ref, f"smallm sym16 m={m} {shape}")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("m,n,k", [(16, 1000, 1920), (40, 300, 4160), (9, 4096, 4096)])
def test_int4_rows(woq, monkeypatch, shape, m, n, k):
    group = 256 if k % 256 == 0 else (128 if k % 128 == 0 else 64)   # the largest dividing K
    plan = _force(woq, monkeypatch, shape, m, n, k, group, True)
    if plan is None:
        pytest.skip(f"shape {shape} does not fit LDS at m={m}")
    _say(f"smallm Int4Linear m={m} n={n} k={k} plan: {plan}")
    seed = 9920 + m + n + k
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    b = workloads.bias(n, seed=seed + 2)
    o = workloads.order(k, seed=seed + 3)
    c, s = woq.quantize_int4_rows(torch.from_numpy(w).cuda())
    cr, sr = oracle.quantize_int4_rows(w)
    ref = oracle.linear_int4_rows(x, oracle.pack_int4(cr), sr, n, k, bias=b, order=o)
    y = woq.linear_int4_rows(to_dev_bf16(x), woq.pack_int4(c), s, bias=torch.from_numpy(b).cuda(),
                             order=torch.from_numpy(o).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_linear(y, ref, f"smallm Int4Linear m={m} {shape}")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("m,n,k", [(5, 100, 96), (16, 1000, 1920), (33, 512, 4160), (64, 640, 2048)])
def test_mxfp4(woq, monkeypatch, shape, m, n, k):
    plan = _force(woq, monkeypatch, shape, m, n, k, 32, False)
    if plan is None:
        pytest.skip(f"shape {shape} does not fit LDS at m={m}")
    _say(f"smallm MXFP4 m={m} n={n} k={k} plan: {plan}")
    seed = 9930 + m + n + k
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    b = workloads.bias(n, seed=seed + 2)
    c, e = woq.quantize_mxfp4(torch.from_numpy(w).cuda())
    cr, er = oracle.quantize_mxfp4(w)
    ref = oracle.linear_mxfp4(x, oracle.pack_uint4(cr), er, n, k, bias=b)
    y = woq.linear_mxfp4(to_dev_bf16(x), woq.pack_uint4(c), e, bias=torch.from_numpy(b).cuda(),
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_linear(y, ref, f"smallm MXFP4 m={m} {shape}")


# Default plans at the edges: 256 K ranges (the split-K pass adds them in
# batches), a single output row (7 of the 8 waves only help load the slice),
# ragged rows and columns with groups of 256.
EDGE = [
    # m, n, k, group
    (16, 100, 262144, 128),
    (64, 1, 4096, 64),
    (20, 17, 8192, 256),
    (8, 300, 16384, 128),
]


@pytest.mark.parametrize("m,n,k,group", EDGE)
def test_default_plan_edges(woq, monkeypatch, m, n, k, group):
    monkeypatch.delenv("WOQ_SM", raising=False)
    plan = woq.linear_plan(m, n, k, group, False)
    assert "path=smallm_lds" in plan, plan
    _say(f"smallm edge m={m} n={n} k={k} g={group} plan: {plan}")
    seed = 9940 + m + n + k
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    b = workloads.bias(n, seed=seed + 2)
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
    qr, sr, zr = oracle.quantize_groups(w, group)
    ref = oracle.linear_int4_groups(x, oracle.pack_uint4(qr), sr, zr, n, k, group, bias=b)
    packed = woq.pack_uint4(q)
    for out in (torch.float32, torch.bfloat16):
        y = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z, bias=torch.from_numpy(b).cuda(), group=group,
                                   out_dtype=out)
        torch.cuda.synchronize()
        check_linear(y, ref, f"smallm edge m={m} n={n} k={k} {out}")
