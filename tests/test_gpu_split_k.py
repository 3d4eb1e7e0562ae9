"""GPU split-K tiled path against the float64 oracle.

linnet "Quantization", std.quant table (linear_int4_groups, dequantize then
linear).  Above 64 rows on narrow layers the tiled GEMM splits K over
workgroups (128 x 256 or 128 x 64 tiles); each K range leaves a float32
partial and a second pass sums them in range order, adds the bias and
converts.  Every weight format goes through it: unsigned groups (byte and
packed zero points, canonical and prepared layouts), signed groups with
float16 scales, Int4Linear rows and MXFP4.  Each case prints its name first.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_linear, to_dev_bf16

pytestmark = pytest.mark.gpu

CASES = [
    # m, n, k, group, bias, order
    (256, 1024, 4096, 128, True, False),   # 8 ranges of 4 steps
    (300, 1000, 4160, 64, True, True),     # ragged rows and columns; the last range holds one step
    (129, 512, 2048, 32, False, True),
    (200, 768, 8192, 256, True, False),
    (96, 1024, 4096, 128, False, False),   # 96 rows on a narrow layer: the small-M kernel declines
    (256, 4096, 4096, 64, True, True),     # 128 x 256 tiles, 8 ranges
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _splits(woq, m, n, k, group, has_order):
    plan = woq.linear_plan(m, n, k, group, has_order)
    fields = dict(f.split("=", 1) for f in plan.split())
    assert fields["path"] == "gemm_mfma" and int(fields["k_splits"]) > 1, plan
    return plan


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order", CASES)
def test_groups(woq, m, n, k, group, with_bias, with_order):
    _say(f"split-K groups m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} "
         f"plan: {_splits(woq, m, n, k, group, with_order)}")
    seed = 9500 + m + n + k
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
        check_linear(y, ref, f"split-K m={m} {out}")
        ys[out] = y
    # the prepared layout feeds the same kernel: bit-identical
    yp = woq.linear_int4_groups_prepared(to_dev_bf16(x), woq.prepare_int4(packed), s, z, bias=dev_b,
                                         order=dev_o, out_dtype=torch.float32)
    # packed zero points: bit-identical to the byte zero points
    zp = woq.pack_zero_points(z)
    yz = woq.linear_int4_groups_zp4(to_dev_bf16(x), packed, s, zp, bias=dev_b, order=dev_o, group=group,
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(yp, ys[torch.float32])
    assert torch.equal(yz, ys[torch.float32])


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order", CASES)
def test_signed_f16_scales(woq, m, n, k, group, with_bias, with_order):
    _say(f"split-K sym16 m={m} n={n} k={k} g={group} plan: {_splits(woq, m, n, k, group, with_order)}")
    seed = 9600 + m + n + k
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
    check_linear(y, ref, f"split-K sym16 m={m}")


@pytest.mark.parametrize("m,n,k", [(256, 1024, 4096), (300, 1000, 4160)])
def test_int4_rows(woq, m, n, k):
    group = 256 if k % 256 == 0 else 64   # the kernels' group for Int4Linear: the largest dividing K
    _say(f"split-K Int4Linear m={m} n={n} k={k} plan: {_splits(woq, m, n, k, group, True)}")
    seed = 9700 + m + n + k
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
    check_linear(y, ref, f"split-K Int4Linear m={m}")


@pytest.mark.parametrize("m,n,k", [(256, 1024, 4096), (129, 512, 2048), (300, 1000, 4160), (256, 4096, 4096)])
def test_mxfp4(woq, m, n, k):
    _say(f"split-K MXFP4 m={m} n={n} k={k} plan: {_splits(woq, m, n, k, 32, False)}")
    seed = 9800 + m + n + k
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    b = workloads.bias(n, seed=seed + 2)
    c, e = woq.quantize_mxfp4(torch.from_numpy(w).cuda())
    cr, er = oracle.quantize_mxfp4(w)
    ref = oracle.linear_mxfp4(x, oracle.pack_uint4(cr), er, n, k, bias=b)
    y = woq.linear_mxfp4(to_dev_bf16(x), woq.pack_uint4(c), e, bias=torch.from_numpy(b).cuda(),
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_linear(y, ref, f"split-K MXFP4 m={m}")
