"""GPU packed 4-bit zero points against the oracle.

linnet "Quantization": Int4GroupLinear's layout is ONNX Runtime's MatMulNBits,
whose zero points are 4-bit values two a byte (R15 in the oracle).  Packing
and unpacking bit-exact (every pair of values, odd group counts); the linear
over packed zero points against the oracle to the linear layer's bar on the
row-streaming, tile GEMV, small-M and GEMM paths, and bit-identical to the
same call with the zero points unpacked.  Each case prints its name first.
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


@pytest.mark.parametrize("n,ng", [(256, 2), (5, 1), (7, 3), (33, 32), (300, 17)])
def test_pack_unpack_bit_exact(woq, n, ng):
    _say(f"zp4 pack/unpack n={n} ng={ng}")
    z = np.random.default_rng(n * ng).integers(0, 16, size=(n, ng)).astype(np.uint8)
    if n == 256 and ng == 2:                      # every pair of values
        a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
        z = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.uint8)
    p = woq.pack_zero_points(torch.from_numpy(z).cuda())
    u = woq.unpack_zero_points(p, ng)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), oracle.pack_zero_points(z))
    assert np.array_equal(u.cpu().numpy(), z)


def test_pack_refuses_out_of_range(woq):
    _say("zp4 pack range")
    z = torch.zeros((3, 5), dtype=torch.uint8, device="cuda")
    z[1, 4] = 16
    with pytest.raises(woq_mod.WoqError) as e:
        woq.pack_zero_points(z)
    assert e.value.status == 5


CASES = [
    # m, n, k, group, bias, order
    (1, 64, 256, 32, False, False),
    (1, 300, 384, 128, True, True),      # 3 groups a row: an odd count
    (3, 4096, 4096, 128, True, False),
    (16, 257, 640, 64, False, True),
    (32, 100, 1280, 256, True, False),   # 5 groups a row
    (130, 300, 384, 128, True, True),
    (256, 512, 4096, 32, False, False),
]


# the tile GEMV (chosen with WOQ_DECODE_MFMA) unpacks the zero points into the
# workspace first; every other path reads them packed
CASES_GEMV = [(1, 300, 384, 128, True, True, "1"), (4, 100, 1280, 256, False, False, "1")]


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order,decode_mfma",
                         [c + ("",) for c in CASES] + CASES_GEMV)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_zp4(woq, monkeypatch, m, n, k, group, with_bias, with_order, decode_mfma, out):
    if decode_mfma:
        monkeypatch.setenv("WOQ_DECODE_MFMA", decode_mfma)
    else:
        monkeypatch.delenv("WOQ_DECODE_MFMA", raising=False)
    plan = woq.linear_plan(m, n, k, group, with_order)
    _say(f"zp4 linear m={m} n={n} k={k} group={group} bias={with_bias} order={with_order} {out} plan: {plan}")
    assert ("path=gemv_mfma" in plan) == bool(decode_mfma)
    seed = m + n + k
    packed, scale, zero = workloads.packed_weights(n, k, group, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    b = workloads.bias(n, seed=seed + 2) if with_bias else None
    o = workloads.order(k, seed=seed + 3) if with_order else None
    zp = oracle.pack_zero_points(zero)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = woq.linear_int4_groups_zp4(to_dev_bf16(x), dev(packed), dev(scale), dev(zp), bias=dev(b), order=dev(o),
                                   group=group, out_dtype=dt)
    y_ref_call = woq.linear_int4_groups(to_dev_bf16(x), dev(packed), dev(scale), dev(zero), bias=dev(b),
                                        order=dev(o), group=group, out_dtype=dt)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref_call)
    check_linear(y, oracle.linear_int4_groups_zp4(x, packed, scale, zp, n, k, group, bias=b, order=o),
                 f"zp4 m={m} n={n} k={k}")


# Row-streaming widths at groups of 64-256, where a wave loads each row's zero
# bytes once and passes them between lanes: rows per workgroup forced with
# WOQ_ROWS_U, odd group counts and partial workgroups.
ROWS_SHARED = [(1, 37, 2432, 128, 16), (1, 45, 8576, 128, 8), (2, 41, 2432, 128, 8), (1, 7, 384, 128, 4),
               (4, 9, 4224, 128, 4), (1, 45, 4160, 64, 16), (2, 23, 2112, 64, 8), (1, 37, 2304, 256, 4),
               (1, 40, 4352, 256, 16)]


@pytest.mark.parametrize("m,n,k,group,u", ROWS_SHARED)
def test_rows_widths_zp4(woq, monkeypatch, m, n, k, group, u):
    monkeypatch.delenv("WOQ_DECODE_MFMA", raising=False)
    monkeypatch.setenv("WOQ_ROWS_U", str(u))
    plan = woq.linear_plan(m, n, k, group, False)
    _say(f"zp4 rows m={m} n={n} k={k} g={group} u={u} plan: {plan}")
    assert "path=rows_dot2" in plan and f"rows_per_group={u} " in plan
    seed = 9100 + m + n + k
    packed, scale, zero = workloads.packed_weights(n, k, group, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 1)
    zp = oracle.pack_zero_points(zero)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = woq.linear_int4_groups_zp4(to_dev_bf16(x), dev(packed), dev(scale), dev(zp), group=group,
                                   out_dtype=torch.float32)
    y_bytes = woq.linear_int4_groups(to_dev_bf16(x), dev(packed), dev(scale), dev(zero), group=group,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y_bytes)
    check_linear(y, oracle.linear_int4_groups_zp4(x, packed, scale, zp, n, k, group), f"zp4 rows m={m} u={u}")
