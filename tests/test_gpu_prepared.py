"""Prepared (fragment-ordered) weights on the GPU.

prepare / unprepare are compared byte for byte with the oracle's definition;
the linear layer over prepared weights is compared with the float64 oracle
and, bit for bit, with the same call over the canonical weights (the kernels
do the same arithmetic and differ only in where they read the bytes).  Each
case prints its name before it touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_linear, to_dev_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("n,k", [(1, 32), (16, 128), (17, 96), (33, 288), (100, 4096), (4096, 4160)])
def test_prepare_matches_oracle_bytes(woq, n, k):
    _say(f"prepare n={n} k={k}")
    rng = np.random.default_rng(n * 7 + k)
    p = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    dp = torch.from_numpy(p).cuda()
    prep = woq.prepare_int4(dp)
    torch.cuda.synchronize()
    expect = oracle.prepare_int4(p, n, k)
    assert prep.numel() == expect.size == woq.prepared_bytes(n, k)
    assert np.array_equal(prep.cpu().numpy(), expect)
    back = woq.unprepare_int4(prep, n, k)
    torch.cuda.synchronize()
    assert torch.equal(back, dp)


def _make(woq, m, n, k, group, seed, with_bias, with_order):
    w = workloads.weight(n, k, seed=seed, std=0.02)
    x = workloads.activations_bf16(m, k, seed=seed + 2)
    b = workloads.bias(n, seed=seed + 3) if with_bias else None
    o = workloads.order(k, seed=seed + 4) if with_order else None
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
    packed = woq.pack_uint4(q)
    dev = dict(x=to_dev_bf16(x), packed=packed, prepared=woq.prepare_int4(packed), scale=s, zero=z,
               bias=None if b is None else torch.from_numpy(b).cuda(),
               order=None if o is None else torch.from_numpy(o).cuda())
    return dev, dict(w=w, x=x, b=b, o=o)


def _ref(host, group, rows=None):
    w = host["w"] if rows is None else host["w"][rows]
    qr, sr, zr = oracle.quantize_groups(w, group)
    b = host["b"]
    if b is not None and rows is not None:
        b = b[rows]
    return oracle.linear_int4_groups(host["x"], oracle.pack_uint4(qr), sr, zr, w.shape[0], w.shape[1],
                                     group, bias=b, order=host["o"])


CASES = [
    # m, n, k, group, bias, order: every path (decode GEMV m <= 4, small-M m <= 32,
    # tiled GEMM above), every group size, ragged n and k
    (1, 64, 256, 32, False, False),
    (1, 100, 96, 32, True, False),
    (1, 48, 4096, 128, False, True),
    (2, 37, 384, 128, True, True),
    (3, 130, 192, 64, False, False),
    (4, 256, 768, 256, True, False),
    (5, 31, 352, 32, False, True),
    (8, 300, 1024, 64, True, False),
    (16, 520, 2048, 32, True, True),
    (17, 200, 512, 128, True, False),
    (28, 300, 1024, 128, False, False),    # two activation tiles
    (64, 1000, 576, 64, False, False),
    (130, 257, 1024, 256, True, True),
    (300, 520, 4096, 128, False, False),
]


@pytest.fixture
def tile_decode(monkeypatch):
    """Canonical weights at m <= 4 on the same tile kernel the prepared layout
    runs on (they would otherwise stream through the row kernel, whose
    float32 rounding order differs): the bitwise comparisons below are about
    the two layouts, not about two kernels."""
    monkeypatch.setenv("WOQ_DECODE_MFMA", "1")


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order", CASES)
def test_linear_prepared(woq, tile_decode, m, n, k, group, with_bias, with_order):
    _say(f"prepared linear m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} "
         f"plan: {woq.linear_plan(m, n, k, group, with_order)}")
    dev, host = _make(woq, m, n, k, group, seed=5000 + m + n + k, with_bias=with_bias,
                      with_order=with_order)
    ref = _ref(host, group)
    for out in (torch.float32, torch.bfloat16):
        y_p = woq.linear_int4_groups_prepared(dev["x"], dev["prepared"], dev["scale"], dev["zero"],
                                              bias=dev["bias"], order=dev["order"], out_dtype=out)
        y_c = woq.linear_int4_groups(dev["x"], dev["packed"], dev["scale"], dev["zero"],
                                     bias=dev["bias"], order=dev["order"], group=group, out_dtype=out)
        torch.cuda.synchronize()
        check_linear(y_p, ref, f"prepared m={m} n={n} k={k} g={group}")
        assert torch.equal(y_p, y_c), "prepared and canonical weights give different bits"


@pytest.mark.parametrize("target,m,n,k,group", [(1, 1, 40, 4096, 128), (6, 1, 48, 2048, 64),
                                                (3, 1, 40, 1536, 32), (1, 4, 64, 4096, 128),
                                                (0, 1, 33, 4160, 64)])
def test_gemv_variants_prepared(woq, tile_decode, monkeypatch, target, m, n, k, group):
    if target:
        monkeypatch.setenv("WOQ_GEMV_WAVES", str(target))
    else:
        monkeypatch.delenv("WOQ_GEMV_WAVES", raising=False)
    _say(f"prepared gemv m={m} n={n} k={k} g={group} plan: {woq.linear_plan(m, n, k, group)}")
    dev, host = _make(woq, m, n, k, group, seed=6000 + n + k, with_bias=True, with_order=False)
    y_p = woq.linear_int4_groups_prepared(dev["x"], dev["prepared"], dev["scale"], dev["zero"],
                                          bias=dev["bias"], out_dtype=torch.float32)
    y_c = woq.linear_int4_groups(dev["x"], dev["packed"], dev["scale"], dev["zero"],
                                 bias=dev["bias"], group=group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_linear(y_p, _ref(host, group), f"prepared gemv m={m} n={n} k={k}")
    assert torch.equal(y_p, y_c)


FULL = list(workloads.DECODE) + list(workloads.ACTORDER) + list(workloads.PREFILL) + \
    [c for c in workloads.SWEEP if c.m in (4, 16, 64) and c.group in (32, 128)]


@pytest.mark.slow
@pytest.mark.parametrize("case", FULL, ids=lambda c: c.name)
def test_full_size_prepared_bitwise(woq, tile_decode, case):
    """At full size the prepared call must reproduce the canonical call bit for
    bit (the canonical call is checked against the oracle by the linear tests);
    a few sampled columns are also checked against the oracle directly."""
    _say(f"prepared full size {case.name} plan: "
         f"{woq.linear_plan(case.m, case.n, case.k, case.group, case.act_order)}")
    w = workloads.weight(case.n, case.k, case.seed_w, outlier_frac=case.outlier_frac,
                         seed_cols=case.seed_cols)
    x = workloads.activations_bf16(case.m, case.k, case.seed_x)
    b = workloads.bias(case.n, case.seed_bias) if case.has_bias else None
    o = workloads.order(case.k, case.seed_order) if case.act_order else None
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), case.group)
    packed = woq.pack_uint4(q)
    del q
    prep = woq.prepare_int4(packed)
    xd = to_dev_bf16(x)
    bd = None if b is None else torch.from_numpy(b).cuda()
    od = None if o is None else torch.from_numpy(o).cuda()
    y_p = woq.linear_int4_groups_prepared(xd, prep, s, z, bias=bd, order=od, out_dtype=torch.float32)
    y_c = woq.linear_int4_groups(xd, packed, s, z, bias=bd, order=od, group=case.group,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_p, y_c)
    rng = np.random.default_rng(case.seed_w)
    rows = np.unique(np.concatenate([[0, case.n - 1], rng.choice(case.n, 16, replace=False)]))
    host = dict(w=w, x=x, b=b, o=o)
    check_linear(y_p[:, torch.from_numpy(rows).cuda()], _ref(host, case.group, rows), case.name)
