"""GPU linear_int4_groups against the float64 oracle.

Small and ragged shapes are compared element by element on every output;
the full-size workloads are compared on sampled output columns that the
oracle evaluates one by one, in the same launch configuration the benchmark
uses.  Each case prints its name before it touches the GPU.
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


def _make(woq, m, n, k, group, seed, with_bias=False, with_order=False, outliers=0.0, std=0.02):
    w = workloads.weight(n, k, seed=seed, std=std, outlier_frac=outliers, seed_cols=seed + 1)
    x = workloads.activations_bf16(m, k, seed=seed + 2)
    b = workloads.bias(n, seed=seed + 3) if with_bias else None
    o = workloads.order(k, seed=seed + 4) if with_order else None
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
    packed = woq.pack_uint4(q)
    dev = dict(x=to_dev_bf16(x), packed=packed, scale=s, zero=z,
               bias=None if b is None else torch.from_numpy(b).cuda(),
               order=None if o is None else torch.from_numpy(o).cuda())
    host = dict(w=w, x=x, b=b, o=o)
    return dev, host


def _ref(host, group, rows=None):
    w = host["w"] if rows is None else host["w"][rows]
    qr, sr, zr = oracle.quantize_groups(w, group)
    pr = oracle.pack_uint4(qr)
    n = w.shape[0]
    return oracle.linear_int4_groups(host["x"], pr, sr, zr, n, w.shape[1], group,
                                     bias=None if host["b"] is None else (host["b"] if rows is None else host["b"][rows]),
                                     order=host["o"])


def _run(woq, dev, group, out_dtype):
    return woq.linear_int4_groups(dev["x"], dev["packed"], dev["scale"], dev["zero"],
                                  bias=dev["bias"], order=dev["order"], group=group,
                                  out_dtype=out_dtype)


SMALL = [
    # m, n, k, group, bias, order
    (1, 64, 256, 32, False, False),      # the tiny workload's shape
    (1, 100, 96, 32, True, False),       # ragged n, k with a 96-wide tail step
    (1, 48, 4096, 128, False, True),
    (2, 37, 384, 128, True, True),
    (3, 130, 192, 64, False, False),
    (4, 256, 768, 256, True, False),
    (5, 31, 352, 32, False, True),
    (8, 300, 1024, 64, True, False),
    (15, 17, 640, 128, False, False),
    (16, 512, 2048, 32, True, True),
    (17, 200, 512, 128, True, False),    # two activation tiles on the small-M path
    (32, 64, 160, 32, False, True),      # last row count on the small-M path, 32-input tail step
    (24, 1000, 1920, 64, True, False),   # 8 waves, several weight tiles per workgroup
    (33, 257, 1024, 256, True, False),   # first row count on the GEMM path
    (64, 1000, 512, 64, False, False),
    (100, 300, 384, 128, True, True),
    (128, 256, 1024, 32, False, False),
    (129, 130, 256, 128, True, False),
    (256, 512, 4096, 128, False, True),
    (200, 33064, 256, 128, True, False),  # the last tile columns in a second launch of 64-row tiles
]


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order", SMALL)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_small_all_outputs(woq, m, n, k, group, with_bias, with_order, out):
    _say(f"linear m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} out={out} "
         f"plan: {woq.linear_plan(m, n, k, group, with_order)}")
    dev, host = _make(woq, m, n, k, group, seed=1000 + m + n + k, with_bias=with_bias,
                      with_order=with_order, outliers=0.01 if with_order else 0.0)
    y = _run(woq, dev, group, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    check_linear(y, _ref(host, group), f"m={m} n={n} k={k} g={group}")


# Tile-GEMV (m <= 4) launch variants: WOQ_GEMV_WAVES sets the planner's
# target number of waves, which at these small sizes forces each steps-per-wave
# class (4, 8, 12/16), one or many waves per workgroup, trailing waves with a
# partial or empty range, group offsets that do not start on a multiple of 4
# and several activation staging batches.
GEMV_VARIANTS = [
    # m, n, k, group, bias, order, target waves, expected "steps_per_wave=.. waves=.."
    (1, 40, 4096, 128, True, False, 1, (16, 2)),
    (1, 17, 1920, 128, False, False, 1, (16, 1)),
    (1, 48, 2048, 64, False, True, 6, (8, 2)),
    (1, 40, 1536, 32, True, False, 3, (12, 1)),
    (1, 40, 4096, 256, False, False, 0, (4, 8)),
    (1, 33, 4160, 64, True, False, 0, (4, 9)),
    (2, 40, 2048, 128, True, False, 6, (8, 2)),
    (3, 50, 3072, 256, False, True, 8, (12, 2)),
    (4, 40, 2048, 32, True, False, 6, (8, 2)),
    (4, 64, 4096, 128, False, False, 1, (16, 2)),
    (4, 31, 1152, 32, True, True, 0, (4, 3)),
]


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order,target,shape", GEMV_VARIANTS)
def test_gemv_launch_variants(woq, monkeypatch, m, n, k, group, with_bias, with_order, target, shape):
    monkeypatch.setenv("WOQ_DECODE_MFMA", "1")   # canonical rows would take the row-streaming kernel
    if target:
        monkeypatch.setenv("WOQ_GEMV_WAVES", str(target))
    else:
        monkeypatch.delenv("WOQ_GEMV_WAVES", raising=False)
    plan = woq.linear_plan(m, n, k, group, with_order)
    _say(f"gemv m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} plan: {plan}")
    assert "path=gemv_mfma" in plan
    assert f"steps_per_wave={shape[0]} " in plan and f"waves={shape[1]} " in plan
    dev, host = _make(woq, m, n, k, group, seed=3000 + m + n + k, with_bias=with_bias,
                      with_order=with_order)
    ref = _ref(host, group)
    for out in (torch.float32, torch.bfloat16):
        y = _run(woq, dev, group, out)
        torch.cuda.synchronize()
        check_linear(y, ref, f"gemv m={m} n={n} k={k} g={group}")


# Small-M path launch variants: WOQ_SKINNY="tiles,cnt" forces the number of
# 16-row weight tiles per workgroup (1, 2, 4: ragged last workgroups included)
# and the steps per wave (partial last waves, ranges that straddle groups,
# 32-input tail steps), with one and two activation tiles per wave and one to
# four wave groups along the rows.
SKINNY_VARIANTS = [
    # m, n, k, group, bias, order, "tiles,cnt", expected (tiles, waves)
    (5, 100, 1024, 128, True, False, "4,2", (4, 4)),
    (16, 70, 2048, 32, False, True, "2,4", (2, 4)),
    (9, 130, 1280, 64, True, False, "4,4", (4, 3)),
    (20, 50, 1536, 256, False, False, "2,6", (2, 2)),
    (32, 33, 864, 32, True, True, "4,2", (4, 4)),
    (12, 64, 4096, 128, False, False, "1,16", (1, 2)),
    (1, 40, 40960, 128, True, False, "4,40", (2, 8)),   # LDS allows 2 tiles, not 4
    # m > 32: wave groups along the activation rows (2 tiles of 16 rows each)
    (33, 70, 1024, 64, True, True, "2,2", (2, 8)),       # 2 groups x 4 K ranges; one row in the last tile
    (64, 100, 2048, 128, False, False, "4,4", (4, 8)),
    (100, 50, 1536, 32, True, False, "1,6", (1, 8)),     # 4 groups x 2 K ranges, ragged rows
    (128, 130, 4096, 256, False, True, "2,16", (2, 8)),
    (80, 40, 768, 128, True, True, "2,4", (2, 6)),       # 3 groups x 2 K ranges
]


@pytest.mark.parametrize("m,n,k,group,with_bias,with_order,override,shape", SKINNY_VARIANTS)
def test_skinny_launch_variants(woq, monkeypatch, m, n, k, group, with_bias, with_order, override, shape):
    monkeypatch.setenv("WOQ_SKINNY", override)
    monkeypatch.setenv("WOQ_FORCE_SKINNY", "1")
    plan = woq.linear_plan(m, n, k, group, with_order)
    _say(f"skinny m={m} n={n} k={k} g={group} bias={with_bias} order={with_order} plan: {plan}")
    assert "path=skinny_mfma" in plan
    assert f"weight_tiles={shape[0]} " in plan and f"waves={shape[1]} " in plan
    dev, host = _make(woq, m, n, k, group, seed=5000 + m + n + k, with_bias=with_bias,
                      with_order=with_order)
    ref = _ref(host, group)
    for out in (torch.float32, torch.bfloat16):
        y = _run(woq, dev, group, out)
        torch.cuda.synchronize()
        check_linear(y, ref, f"skinny m={m} n={n} k={k} g={group}")


def test_tiny_workload(woq):
    c = workloads.TINY
    _say(f"tiny workload {c.name}")
    dev, host = _make(woq, c.m, c.n, c.k, c.group, seed=0)
    # use the registry seeds for the weight and activations
    host["w"] = workloads.weight(c.n, c.k, c.seed_w)
    host["x"] = workloads.activations_bf16(c.m, c.k, c.seed_x)
    q, s, z = woq.quantize_groups(torch.from_numpy(host["w"]).cuda(), c.group)
    dev.update(x=to_dev_bf16(host["x"]), packed=woq.pack_uint4(q), scale=s, zero=z)
    for dt in (torch.float32, torch.bfloat16):
        check_linear(_run(woq, dev, c.group, dt), _ref(host, c.group), "tiny")


def test_order_is_a_gather_bit_for_bit(woq):
    for m, n, k, g in ((1, 96, 1024, 128), (4, 64, 512, 32), (48, 128, 768, 64)):
        _say(f"order invariants m={m} n={n} k={k} g={g}")
        dev, host = _make(woq, m, n, k, g, seed=77 + m, with_order=True)
        y_ord = _run(woq, dev, g, torch.float32)
        xg = host["x"][:, host["o"]]
        y_pre = woq.linear_int4_groups(to_dev_bf16(xg), dev["packed"], dev["scale"], dev["zero"],
                                       group=g, out_dtype=torch.float32)
        assert torch.equal(y_ord, y_pre)
        ident = torch.arange(k, dtype=torch.int32, device="cuda")
        y_id = woq.linear_int4_groups(dev["x"], dev["packed"], dev["scale"], dev["zero"],
                                      order=ident, group=g, out_dtype=torch.float32)
        y_no = woq.linear_int4_groups(dev["x"], dev["packed"], dev["scale"], dev["zero"],
                                      group=g, out_dtype=torch.float32)
        assert torch.equal(y_id, y_no)


def test_deterministic(woq):
    for m in (1, 16, 200):
        _say(f"determinism m={m}")
        dev, _ = _make(woq, m, 1024, 2048, 128, seed=5)
        a = _run(woq, dev, 128, torch.float32)
        b = _run(woq, dev, 128, torch.float32)
        assert torch.equal(a, b)


def test_degenerate_sizes(woq):
    _say("degenerate sizes")
    dev, host = _make(woq, 3, 40, 64, 32, seed=9, with_bias=True)
    # m == 0 and n == 0: nothing to do
    x0 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    y0 = woq.linear_int4_groups(x0, dev["packed"], dev["scale"], dev["zero"], group=32)
    assert y0.shape == (0, 40)
    # k == 0: the bias alone
    lib = woq.load()
    y = torch.full((3, 40), 7.0, dtype=torch.float32, device="cuda")
    assert lib.woq_linear_int4_groups(None, 3, None, None, None, dev["bias"].data_ptr(), None, 40, 0, 32, 0,
                                      y.data_ptr(), None, 0, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(y, dev["bias"].expand(3, 40))
    assert lib.woq_linear_int4_groups(None, 3, None, None, None, None, None, 40, 0, 32, 0,
                                      y.data_ptr(), None, 0, None) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    # all-zero weights give exactly the bias
    q, s, z = woq.quantize_groups(torch.zeros((40, 64), device="cuda"), 32)
    yb = woq.linear_int4_groups(dev["x"], woq.pack_uint4(q), s, z, bias=dev["bias"], group=32,
                                out_dtype=torch.float32)
    assert torch.equal(yb, dev["bias"].expand(3, 40))


def test_graph_replay_matches_eager(woq):
    for m, n, k, g, with_order in ((1, 4096, 4096, 128, False), (16, 1024, 4096, 32, True),
                                   (256, 1024, 2048, 128, False)):
        _say(f"graph replay m={m} n={n} k={k} g={g}")
        dev, _ = _make(woq, m, n, k, g, seed=31 + m, with_bias=True, with_order=with_order)
        eager = _run(woq, dev, g, torch.bfloat16).clone()
        ws_bytes = woq.linear_workspace_bytes(m, n, k, g, with_order)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            woq.linear_int4_groups(dev["x"], dev["packed"], dev["scale"], dev["zero"], bias=dev["bias"],
                                   order=dev["order"], group=g, out=out, out_dtype=torch.bfloat16,
                                   workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            woq.linear_int4_groups(dev["x"], dev["packed"], dev["scale"], dev["zero"], bias=dev["bias"],
                                   order=dev["order"], group=g, out=out, out_dtype=torch.bfloat16,
                                   workspace=ws)
        for rep in range(4):
            out.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {rep} differs"


# ---------------------------------------------------------------------------
# Full-size workloads: sampled output columns
# ---------------------------------------------------------------------------

def _sample_rows(n, seed, count=48):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, n - 1, n // 2], rng.choice(n, count, replace=False)]))
    return rows


FULL = (list(workloads.DECODE) + list(workloads.PREFILL) + list(workloads.ACTORDER) + list(workloads.SWEEP)
        + list(workloads.MIDSIZE) + list(workloads.SMALLBATCH) + list(workloads.FEWROWS))


@pytest.mark.slow
@pytest.mark.parametrize("case", FULL, ids=lambda c: c.name)
def test_full_size_sampled(woq, case):
    _say(f"full size {case.name} plan: {woq.linear_plan(case.m, case.n, case.k, case.group, case.act_order)}")
    w = workloads.weight(case.n, case.k, case.seed_w, outlier_frac=case.outlier_frac,
                         seed_cols=case.seed_cols)
    x = workloads.activations_bf16(case.m, case.k, case.seed_x)
    b = workloads.bias(case.n, case.seed_bias) if case.has_bias else None
    o = workloads.order(case.k, case.seed_order) if case.act_order else None
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), case.group)
    packed = woq.pack_uint4(q)
    del q
    y = woq.linear_int4_groups(to_dev_bf16(x), packed, s, z,
                               bias=None if b is None else torch.from_numpy(b).cuda(),
                               order=None if o is None else torch.from_numpy(o).cuda(),
                               group=case.group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    rows = _sample_rows(case.n, case.seed_w)
    host = dict(w=w[rows], x=x, b=None if b is None else b[rows], o=o)
    y_ref = _ref(host, case.group)
    check_linear(y[:, torch.from_numpy(rows).cuda()], y_ref, case.name)
