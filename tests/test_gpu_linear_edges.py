"""GPU linear layer on the edge cases of its inputs, on every kernel path.

Each case runs on the row-streaming decode path (m <= 4), the tile GEMV
(m <= 4 with WOQ_DECODE_MFMA), the small-M MFMA path (5 <= m <= 64, and
m = 100 with its launch shape forced), the small-M path with the activation
slice in LDS (16 <= m <= 64 on narrow layers, and m = 5 with its launch shape
forced) and the tiled GEMM (m > 64), and is
compared with the float64 oracle to the same
gate as every other parity test:

* a gather index that repeats some inputs and skips others (the `order`
  argument only has to hold in-range indices; linnet "Quantization",
  std.quant table, order [In; i32]);
* activations with 1 % of the input channels scaled by 50 (the salient
  channels activation-aware scaling is built on: "20. Quantization",
  "Stretch exercises"), and activations with a large common offset, which
  the kernels' fold s * (sum x (128 + q) - (128 + z) * sum x) must cancel
  without losing the signal;
* group scales that are float32 subnormals, and scales near 2^100.

Also the row-streaming kernel's launch variants: forced rows per workgroup
(4, 8, 16), one to sixteen waves (K up to 32768), a chunk whose tail lanes lie
past K, ragged output counts and every activation row count.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_linear, to_dev_bf16

pytestmark = pytest.mark.gpu

# (m, n, k, group, env) per kernel path
PATHS = {
    "rows": [(1, 300, 2048, 128, {}), (3, 100, 1536, 64, {})],
    "gemv": [(1, 300, 2048, 128, {"WOQ_DECODE_MFMA": "1"}), (4, 100, 1024, 32, {"WOQ_DECODE_MFMA": "1"})],
    "skinny": [(16, 200, 2048, 128, {"WOQ_SM": "0"}), (7, 64, 1024, 32, {}), (64, 300, 1024, 128, {"WOQ_SM": "0"}),
               (100, 300, 1024, 128, {"WOQ_SKINNY": "2,4"})],
    "smallm": [(16, 200, 2048, 128, {}), (64, 300, 1024, 128, {}), (24, 1000, 8192, 32, {}),
               (5, 100, 1024, 64, {"WOQ_SM": "2,4"})],
    "gemm": [(100, 300, 1024, 128, {}), (160, 256, 512, 256, {})],
}
CASES = [(path, *c) for path, cs in PATHS.items() for c in cs]
PATH_TAG = {"rows": "rows_dot2", "gemv": "gemv_mfma", "skinny": "skinny_mfma", "smallm": "smallm_lds",
            "gemm": "gemm_mfma"}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _env(monkeypatch, env):
    monkeypatch.delenv("WOQ_DECODE_MFMA", raising=False)
    monkeypatch.delenv("WOQ_ROWS_U", raising=False)
    monkeypatch.delenv("WOQ_SKINNY", raising=False)
    monkeypatch.delenv("WOQ_SM", raising=False)
    for key, val in env.items():
        monkeypatch.setenv(key, val)


def _quantized(woq, n, k, group, seed):
    w = workloads.weight(n, k, seed=seed)
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
    return w, woq.pack_uint4(q), s, z


def _oracle_from_weight(w, x, group, bias=None, order=None):
    qr, sr, zr = oracle.quantize_groups(w, group)
    return oracle.linear_int4_groups(x, oracle.pack_uint4(qr), sr, zr, w.shape[0], w.shape[1], group,
                                     bias=bias, order=order)


def _check_path(woq, path, m, n, k, group, order):
    plan = woq.linear_plan(m, n, k, group, order is not None)
    assert f"path={PATH_TAG[path]}" in plan, plan
    return plan


@pytest.mark.parametrize("path,m,n,k,group,env", CASES)
def test_order_with_repeated_indices(woq, monkeypatch, path, m, n, k, group, env):
    _env(monkeypatch, env)
    _say(f"repeated-index order {path} m={m} n={n} k={k} g={group}")
    _check_path(woq, path, m, n, k, group, True)
    seed = 8100 + m + n + k
    w, packed, s, z = _quantized(woq, n, k, group, seed)
    x = workloads.activations_bf16(m, k, seed + 1)
    o = workloads.order_with_repeats(k, seed + 2)
    assert len(np.unique(o)) < k
    b = workloads.bias(n, seed + 3)
    ref = _oracle_from_weight(w, x, group, bias=b, order=o)
    for out in (torch.float32, torch.bfloat16):
        y = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z, bias=torch.from_numpy(b).cuda(),
                                   order=torch.from_numpy(o).cuda(), group=group, out_dtype=out)
        torch.cuda.synchronize()
        check_linear(y, ref, f"{path} repeated order m={m}")
    # the gather equals running on the gathered activations
    xg = x[:, o]
    y_ord = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z, order=torch.from_numpy(o).cuda(), group=group,
                                   out_dtype=torch.float32)
    y_pre = woq.linear_int4_groups(to_dev_bf16(xg), packed, s, z, group=group, out_dtype=torch.float32)
    assert torch.equal(y_ord, y_pre)


@pytest.mark.parametrize("kind", ["outliers_x50", "offset_32"])
@pytest.mark.parametrize("path,m,n,k,group,env", CASES)
def test_activation_distributions(woq, monkeypatch, kind, path, m, n, k, group, env):
    _env(monkeypatch, env)
    _say(f"activations {kind} {path} m={m} n={n} k={k} g={group}")
    _check_path(woq, path, m, n, k, group, False)
    seed = 8300 + m + n + k
    w, packed, s, z = _quantized(woq, n, k, group, seed)
    if kind == "outliers_x50":
        x = workloads.activations_bf16(m, k, seed + 1, outlier_frac=0.01, outlier_mult=50.0, seed_cols=seed + 5)
    else:
        x = workloads.activations_bf16(m, k, seed + 1, offset=32.0)
    ref = _oracle_from_weight(w, x, group)
    for out in (torch.float32, torch.bfloat16):
        y = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z, group=group, out_dtype=out)
        torch.cuda.synchronize()
        check_linear(y, ref, f"{path} {kind} m={m}")


@pytest.mark.parametrize("kind", ["subnormal", "huge"])
@pytest.mark.parametrize("path,m,n,k,group,env", CASES)
def test_extreme_group_scales(woq, monkeypatch, kind, path, m, n, k, group, env):
    """Scales written directly (the quantizer never makes them): float32
    subnormals in [2^-135, 2^-134) or values in [2^100, 2^101), with random
    codes and zero points."""
    _env(monkeypatch, env)
    _say(f"scales {kind} {path} m={m} n={n} k={k} g={group}")
    _check_path(woq, path, m, n, k, group, False)
    rng = np.random.default_rng(8500 + m + n + k)
    ng = k // group
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    zero = rng.integers(0, 16, size=(n, ng), dtype=np.uint8)
    frac = rng.uniform(1.0, 2.0, size=(n, ng))
    exp = -135 if kind == "subnormal" else 100
    scale = (frac * 2.0 ** exp).astype(np.float32)
    if kind == "subnormal":
        assert np.all(scale < np.finfo(np.float32).tiny) and np.all(scale > 0)
    x = workloads.activations_bf16(m, k, 8600 + m)
    ref = oracle.linear_int4_groups(x, packed, scale, zero, n, k, group)
    dev = [torch.from_numpy(a).cuda() for a in (packed, scale, zero)]
    for out in (torch.float32, torch.bfloat16):
        y = woq.linear_int4_groups(to_dev_bf16(x), *dev, group=group, out_dtype=out)
        torch.cuda.synchronize()
        check_linear(y, ref, f"{path} {kind} scales m={m}")


# Row-streaming kernel launch variants: rows per workgroup forced with
# WOQ_ROWS_U (at most 8 when m = 2, always 4 when m > 2); waves = ceil(K / 2048).
ROWS_VARIANTS = [
    # m, n, k, group, bias, order, rows per workgroup, expected waves
    (1, 37, 64, 32, True, False, 4, 1),        # one chunk, most lanes past K
    (1, 100, 2080, 32, False, True, 8, 2),     # second chunk holds 32 inputs
    (1, 257, 4096, 128, True, False, 16, 2),
    (2, 70, 6144, 64, True, True, 16, 3),
    (2, 33, 14336, 256, False, False, 8, 7),
    (3, 50, 3072, 128, True, False, 4, 2),     # three rows computed as four
    (4, 64, 2048, 32, False, True, 4, 1),
    (4, 19, 32768, 128, True, False, 4, 16),   # the longest rows this path takes
    (1, 1000, 30720, 256, False, False, 16, 15),
    (2, 5, 256, 128, True, False, 8, 1),       # fewer rows than one workgroup
    # groups of 64-256: a wave loads each (scale, zero) pair once for its lanes
    (1, 45, 4160, 64, True, False, 16, 3),     # 65 groups a row, the last chunk holds one
    (1, 37, 2304, 256, False, True, 4, 2),     # 9 groups a row: more rows per load than rows
    (2, 19, 4352, 256, True, False, 8, 3),
    (1, 37, 2432, 128, True, True, 8, 2),      # second chunk holds 3 groups
    (2, 41, 2432, 128, False, False, 8, 2),
    (1, 45, 8576, 128, False, True, 16, 5),    # 67 groups a row, 45 rows: a partial workgroup
    (1, 7, 128, 128, True, False, 4, 1),       # one group
]


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order,u,waves", ROWS_VARIANTS)
def test_rows_launch_variants(woq, monkeypatch, m, n, k, group, with_bias, with_order, u, waves):
    _env(monkeypatch, {"WOQ_ROWS_U": str(u)})
    plan = woq.linear_plan(m, n, k, group, with_order)
    _say(f"rows m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} plan: {plan}")
    assert "path=rows_dot2" in plan
    expect_u = u if m == 1 else (min(u, 8) if m == 2 else 4)
    assert f"rows_per_group={expect_u} " in plan and f"waves={waves} " in plan
    seed = 8700 + m + n + k
    w, packed, s, z = _quantized(woq, n, k, group, seed)
    x = workloads.activations_bf16(m, k, seed + 1)
    b = workloads.bias(n, seed + 2) if with_bias else None
    o = workloads.order(k, seed + 3) if with_order else None
    ref = _oracle_from_weight(w, x, group, bias=b, order=o)
    for out in (torch.float32, torch.bfloat16):
        y = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z, bias=None if b is None else torch.from_numpy(b).cuda(),
                                   order=None if o is None else torch.from_numpy(o).cuda(), group=group,
                                   out_dtype=out)
        torch.cuda.synchronize()
        check_linear(y, ref, f"rows m={m} n={n} k={k} g={group}")


def test_rows_matches_tile_gemv(woq, monkeypatch):
    """The two decode kernels agree on the same call to float32 rounding."""
    for m, n, k, g in ((1, 4096, 4096, 128), (2, 1024, 4096, 32), (4, 512, 14336, 64)):
        _say(f"rows vs gemv m={m} n={n} k={k} g={g}")
        w, packed, s, z = _quantized(woq, n, k, g, 8900 + m)
        x = to_dev_bf16(workloads.activations_bf16(m, k, 8901 + m))
        _env(monkeypatch, {})
        a = woq.linear_int4_groups(x, packed, s, z, group=g, out_dtype=torch.float32)
        _env(monkeypatch, {"WOQ_DECODE_MFMA": "1"})
        b = woq.linear_int4_groups(x, packed, s, z, group=g, out_dtype=torch.float32)
        torch.cuda.synchronize()
        scale = float(a.abs().max())
        assert float((a - b).abs().max()) <= 1e-5 * scale


# Small-M activations through the fragment-order pre-pass (WOQ_SKINNY_XFRAG=1)
# and straight from x (=0): the same bf16 values meet the same weight
# fragments in the same order, so the outputs are bit-identical; both are
# checked against the oracle too.  Unsigned codes, signed float16-scale codes
# and MXFP4, with and without the act-order gather.
XFRAG_CASES = [
    # m, n, k, group, bias, order, format
    (17, 100, 1024, 128, True, False, "u4"),
    (24, 64, 2048, 32, False, True, "u4"),
    (33, 70, 1536, 64, True, True, "u4"),
    (48, 130, 4096, 256, False, False, "u4"),
    (64, 50, 768, 128, True, True, "u4"),
    (40, 96, 1024, 32, True, False, "sym16"),
    (56, 80, 2048, 32, False, False, "mx"),
]


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order,fmt", XFRAG_CASES)
def test_skinny_fragment_prepass(woq, monkeypatch, m, n, k, group, with_bias, with_order, fmt):
    _env(monkeypatch, {"WOQ_SM": "0"})   # these narrow layers would otherwise take the LDS small-M path
    seed = 9100 + m + n + k
    x = workloads.activations_bf16(m, k, seed + 1)
    b = workloads.bias(n, seed + 2) if with_bias else None
    o = workloads.order(k, seed + 3) if with_order and fmt != "mx" else None
    w = workloads.weight(n, k, seed=seed)
    wd = torch.from_numpy(w).cuda()
    if fmt == "u4":
        q, s, z = woq.quantize_groups(wd, group)
        packed = woq.pack_uint4(q)
        qr, sr, zr = oracle.quantize_groups(w, group)
        ref = oracle.linear_int4_groups(x, oracle.pack_uint4(qr), sr, zr, n, k, group, bias=b, order=o)
        call = lambda out: woq.linear_int4_groups(
            to_dev_bf16(x), packed, s, z, bias=None if b is None else torch.from_numpy(b).cuda(),
            order=None if o is None else torch.from_numpy(o).cuda(), group=group, out_dtype=out)
    elif fmt == "sym16":
        c, s16 = woq.quantize_int4_sym(wd, group)
        packed = woq.pack_int4(c)
        cr, sr = oracle.quantize_int4_sym_f16(w, group)
        ref = oracle.linear_int4_sym_f16(x, oracle.pack_int4(cr), sr, n, k, group, bias=b)
        call = lambda out: woq.linear_int4_sym(to_dev_bf16(x), packed, s16,
                                               bias=None if b is None else torch.from_numpy(b).cuda(),
                                               group=group, out_dtype=out)
    else:
        codes, scales = woq.quantize_mxfp4(wd)
        blocks = woq.pack_uint4(codes)
        cr, sr = oracle.quantize_mxfp4(w)
        ref = oracle.linear_mxfp4(x, oracle.pack_uint4(cr), sr, n, k, bias=b)
        call = lambda out: woq.linear_mxfp4(to_dev_bf16(x), blocks, scales,
                                            bias=None if b is None else torch.from_numpy(b).cuda(), out_dtype=out)
    outs = {}
    for flag in ("1", "0"):
        monkeypatch.setenv("WOQ_SKINNY_XFRAG", flag)
        plan = woq.linear_plan(m, n, k, 32 if fmt == "mx" else group, o is not None)
        _say(f"xfrag={flag} {fmt} m={m} n={n} k={k} g={group} plan: {plan}")
        assert "path=skinny_mfma" in plan and (("fragments" in plan) == (flag == "1")), plan
        outs[flag] = {dt: call(dt) for dt in (torch.float32, torch.bfloat16)}
        torch.cuda.synchronize()
    for dt in (torch.float32, torch.bfloat16):
        assert torch.equal(outs["1"][dt], outs["0"][dt])
        check_linear(outs["1"][dt], ref, f"xfrag {fmt} m={m} n={n} k={k} g={group}")
