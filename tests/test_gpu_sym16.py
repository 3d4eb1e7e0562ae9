"""GPU signed int4 groups with float16 scales against the float64 oracle.

The format of tinyllm L8.5 ("Quantization: int8, int4 group (packed), fp8, KV
quant", section 2, "int4 per group" and "Packing"): the quantizer, packing and
dequantization bit for bit; the linear layer on every path (decode GEMV,
small-M, tiled GEMM, prepared weights) to the same bar as the unsigned layout.
Each case prints its name before it touches the GPU.
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


def _codes_scale(woq, w, group):
    c, s = woq.quantize_int4_sym(torch.from_numpy(w).cuda(), group)
    torch.cuda.synchronize()
    return c, s


# ---------------------------------------------------------------------------
# Quantize, pack, unpack, dequantize: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,group,std", [(64, 256, 32, 0.02), (37, 96, 32, 1.0), (16, 512, 16, 30.0),
                                           (8, 128, 64, 1e-3), (5, 64, 2, 0.5)])
def test_quantize_matches_oracle(woq, n, k, group, std):
    _say(f"sym16 quantize n={n} k={k} g={group} std={std}")
    rng = np.random.default_rng(n * 1000 + k)
    w = (rng.standard_normal((n, k)) * std).astype(np.float32)
    w[0, :group] = 0.0                                  # an all-zero group
    w[1, group:2 * group] = 3e-6                        # a float16-subnormal scale
    if n > 2:
        w[2, :group] = 1e-9                             # underflows float16: codes 0
    if k >= 3 * group:                                  # exact ties against the stored scale
        w[1, 2 * group:3 * group] = 0.0
        w[1, 2 * group] = 7.0021
        w[1, 2 * group + 1] = 3.5
        w[1, 2 * group + 2] = -2.5
    c, s = _codes_scale(woq, w, group)
    c_ref, s_ref = oracle.quantize_int4_sym_f16(w, group)
    assert np.array_equal(c.cpu().numpy(), c_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))


def test_quantize_refuses_overflow_and_nan(woq):
    _say("sym16 quantize errors")
    big = torch.full((2, 64), 1e6, dtype=torch.float32, device="cuda")   # 1e6 / 7 overflows float16
    with pytest.raises(woq_mod.WoqError) as e:
        woq.quantize_int4_sym(big, 32)
    assert e.value.status == 5
    bad = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    bad[1, 3] = float("nan")
    with pytest.raises(woq_mod.WoqError) as e:
        woq.quantize_int4_sym(bad, 32)
    assert e.value.status == 4


def test_pack_unpack_every_pair(woq):
    _say("sym16 pack/unpack all pairs")
    pairs = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], dtype=np.int8)
    p = woq.pack_int4(torch.from_numpy(pairs.copy()).cuda())
    assert np.array_equal(p.cpu().numpy(), oracle.pack_int4(pairs))
    every = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(256, 1).cuda()
    u = woq.unpack_int4(every)
    assert np.array_equal(u.cpu().numpy(), oracle.unpack_int4(every.cpu().numpy()))
    with pytest.raises(woq_mod.WoqError) as e:
        woq.pack_int4(torch.tensor([[8, 0]], dtype=torch.int8, device="cuda"))
    assert e.value.status == 5


@pytest.mark.parametrize("n,k,group", [(64, 256, 32), (33, 192, 64), (7, 512, 256)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bit_exact(woq, n, k, group, out):
    _say(f"sym16 dequantize n={n} k={k} g={group} {out}")
    w = workloads.weight(n, k, seed=n + k)
    c, s = _codes_scale(woq, w, group)
    packed = woq.pack_int4(c)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    got = woq.dequantize_int4_sym(packed, s, group, out_dtype=dt)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.quantize_int4_sym_f16(w, group)
    want = oracle.dequantize_int4_sym_f16(oracle.pack_int4(c_ref), s_ref, n, k, group, out=out)
    g = got.cpu()
    g = g.numpy() if out == "f32" else g.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(g, want)


# ---------------------------------------------------------------------------
# Linear layer on every path
# ---------------------------------------------------------------------------

def _make(woq, m, n, k, group, seed, with_bias=False, with_order=False):
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed=seed + 2)
    b = workloads.bias(n, seed=seed + 3) if with_bias else None
    o = workloads.order(k, seed=seed + 4) if with_order else None
    c, s = _codes_scale(woq, w, group)
    dev = dict(x=to_dev_bf16(x), packed=woq.pack_int4(c), scale=s,
               bias=None if b is None else torch.from_numpy(b).cuda(),
               order=None if o is None else torch.from_numpy(o).cuda())
    return dev, dict(w=w, x=x, b=b, o=o)


def _ref(host, group, rows=None):
    w = host["w"] if rows is None else host["w"][rows]
    c, s = oracle.quantize_int4_sym_f16(w, group)
    b = host["b"]
    if b is not None and rows is not None:
        b = b[rows]
    return oracle.linear_int4_sym_f16(host["x"], oracle.pack_int4(c), s, w.shape[0], w.shape[1], group,
                                      bias=b, order=host["o"])


SMALL = [
    # m, n, k, group, bias, order (paths: decode m <= 4, small-M m <= 32, tiled above)
    (1, 64, 256, 32, False, False),
    (1, 100, 96, 32, True, False),
    (2, 48, 4096, 128, False, True),
    (4, 256, 768, 256, True, False),
    (1, 40, 384, 64, False, False),
    (5, 31, 352, 32, False, True),
    (16, 512, 2048, 32, True, True),
    (24, 1000, 1920, 64, True, False),
    (32, 64, 160, 32, False, False),
    (33, 257, 1024, 256, True, False),
    (100, 300, 384, 128, True, True),
    (256, 512, 1024, 32, False, False),
    (200, 33064, 256, 128, True, False),
]


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order", SMALL)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_small(woq, m, n, k, group, with_bias, with_order, out):
    _say(f"sym16 linear m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} {out} "
         f"plan: {woq.linear_plan(m, n, k, group, with_order)}")
    dev, host = _make(woq, m, n, k, group, seed=m * 7 + n, with_bias=with_bias, with_order=with_order)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = woq.linear_int4_sym(dev["x"], dev["packed"], dev["scale"], bias=dev["bias"], order=dev["order"],
                            group=group, out_dtype=dt)
    torch.cuda.synchronize()
    check_linear(y, _ref(host, group), f"sym16 m={m} n={n} k={k} g={group}")


@pytest.mark.parametrize("m,n,k,group", [(1, 100, 1024, 32), (3, 64, 4096, 128), (16, 300, 512, 64),
                                         (130, 256, 640, 128)])
def test_linear_prepared_is_bit_identical(woq, monkeypatch, m, n, k, group):
    monkeypatch.setenv("WOQ_DECODE_MFMA", "1")   # the canonical call on the prepared layout's tile kernel
    _say(f"sym16 prepared m={m} n={n} k={k} g={group}")
    dev, host = _make(woq, m, n, k, group, seed=m + n + k, with_bias=True)
    y = woq.linear_int4_sym(dev["x"], dev["packed"], dev["scale"], bias=dev["bias"], group=group,
                            out_dtype=torch.float32)
    prep = woq.prepare_int4(dev["packed"])
    yp = woq.linear_int4_sym(dev["x"], prep, dev["scale"], bias=dev["bias"], group=group,
                             out_dtype=torch.float32, prepared=True)
    torch.cuda.synchronize()
    assert torch.equal(y, yp)
    check_linear(yp, _ref(host, group), f"sym16 prepared m={m}")


@pytest.mark.parametrize("g", [32, 128, 256])
def test_signed_equals_unsigned_with_zero_point_eight(woq, g):
    """A signed code c is the unsigned code c + 8 with zero point 8: the two
    entry points must agree bit for bit on the same weights, on every path."""
    _say(f"sym16 vs unsigned zero 8 g={g}")
    rng = np.random.default_rng(9 + g)
    n, k = 96, 1024
    c = torch.from_numpy(rng.integers(-8, 8, size=(n, k)).astype(np.int8)).cuda()
    s16 = torch.from_numpy(rng.uniform(0.001, 0.01, size=(n, k // g)).astype(np.float16)).cuda()
    packed_s = woq.pack_int4(c)
    packed_u = woq.pack_uint4((c.to(torch.int16) + 8).to(torch.uint8))
    zero = torch.full((n, k // g), 8, dtype=torch.uint8, device="cuda")
    for m in (1, 4, 16, 64, 200):
        x = to_dev_bf16(workloads.activations_bf16(m, k, seed=m))
        ys = woq.linear_int4_sym(x, packed_s, s16, group=g, out_dtype=torch.float32)
        yu = woq.linear_int4_groups(x, packed_u, s16.float(), zero, group=g, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(ys, yu), m


# Row-streaming widths (WOQ_ROWS_U) at groups of 64-256, where a wave loads
# each row's float16 scales once and passes them between lanes.
ROWS_SHARED = [(1, 37, 2432, 128, 16), (1, 45, 4160, 64, 16), (2, 23, 2304, 256, 8), (1, 40, 8576, 128, 8),
               (3, 9, 640, 128, 4)]


@pytest.mark.parametrize("m,n,k,group,u", ROWS_SHARED)
def test_rows_widths(woq, monkeypatch, m, n, k, group, u):
    monkeypatch.delenv("WOQ_DECODE_MFMA", raising=False)
    monkeypatch.setenv("WOQ_ROWS_U", str(u))
    plan = woq.linear_plan(m, n, k, group, False)
    _say(f"sym16 rows m={m} n={n} k={k} g={group} u={u} plan: {plan}")
    assert "path=rows_dot2" in plan and f"rows_per_group={u} " in plan
    dev, host = _make(woq, m, n, k, group, seed=500 + m + n, with_bias=True)
    y = woq.linear_int4_sym(dev["x"], dev["packed"], dev["scale"], bias=dev["bias"], group=group,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_linear(y, _ref(host, group), f"sym16 rows m={m} u={u}")


FULL = [(1, 14336, 4096, 32), (1, 4096, 14336, 32), (16, 14336, 4096, 32), (2048, 4096, 4096, 32)]


@pytest.mark.slow
@pytest.mark.parametrize("m,n,k,group", FULL)
def test_full_size_sampled(woq, m, n, k, group):
    _say(f"sym16 full size m={m} n={n} k={k} g={group} plan: {woq.linear_plan(m, n, k, group)}")
    dev, host = _make(woq, m, n, k, group, seed=130 + m, with_bias=True)
    y = woq.linear_int4_sym(dev["x"], dev["packed"], dev["scale"], bias=dev["bias"], group=group,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([[0, n - 1, n // 2], rng.choice(n, 48, replace=False)]))
    check_linear(y[:, torch.from_numpy(rows).cuda()], _ref(host, group, rows), f"sym16 full m={m}")
