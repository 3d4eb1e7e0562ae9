"""The allocation-free linear entry point against the one with a caller workspace.

woq_linear_int4_groups_noalloc runs the same kernels as woq_linear_int4_groups
with the library's own device array as workspace, for callers that cannot
allocate.  Two calls in a row (the second on a smaller input, so the array
holds the first call's leftovers) must each equal the workspace call bit for
bit, and pass the oracle's gate; a size whose workspace exceeds the array is
refused before anything runs.  Called through the C ABI.
"""
import ctypes
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


def _case(woq, m, n, k, group, seed, with_order):
    w = workloads.weight(n, k, seed=seed)
    x = workloads.activations_bf16(m, k, seed + 1)
    b = workloads.bias(n, seed + 2)
    o = workloads.order(k, seed + 3) if with_order else None
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
    dev = dict(x=to_dev_bf16(x), packed=woq.pack_uint4(q), scale=s, zero=z, bias=torch.from_numpy(b).cuda(),
               order=None if o is None else torch.from_numpy(o).cuda())
    qr, sr, zr = oracle.quantize_groups(w, group)
    ref = oracle.linear_int4_groups(x, oracle.pack_uint4(qr), sr, zr, n, k, group, bias=b, order=o)
    return dev, ref


def _ptr(t):
    return None if t is None else t.data_ptr()


def _noalloc(lib, dev, m, n, k, group, out):
    stream = torch.cuda.current_stream().cuda_stream
    return lib.woq_linear_int4_groups_noalloc(_ptr(dev["x"]), m, _ptr(dev["packed"]), _ptr(dev["scale"]),
                                              _ptr(dev["zero"]), _ptr(dev["bias"]), _ptr(dev["order"]), n, k,
                                              group, 0 if out.dtype == torch.float32 else 1, _ptr(out), stream)


def _with_workspace(lib, dev, m, n, k, group, out):
    need = lib.woq_linear_workspace_bytes(m, n, k, group, int(dev["order"] is not None))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.woq_linear_int4_groups(_ptr(dev["x"]), m, _ptr(dev["packed"]), _ptr(dev["scale"]), _ptr(dev["zero"]),
                                    _ptr(dev["bias"]), _ptr(dev["order"]), n, k, group,
                                    0 if out.dtype == torch.float32 else 1, _ptr(out), _ptr(ws) if need else None,
                                    need, stream)
    return st, need


# (m, n, k, group, order): the first call uses the tiled GEMM's workspace (the
# reordered activations, group sums and scale table); the second is smaller.
SEQUENCES = [
    [(100, 1000, 2048, 128, True), (40, 300, 1024, 64, False)],
    [(300, 4096, 4096, 128, False), (3, 4096, 4096, 128, True)],   # a split over K, then the row kernel
    [(20, 2000, 4096, 32, True), (1, 1024, 4096, 128, True)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "_then_".join(f"{c[0]}x{c[1]}x{c[2]}" for c in s))
def test_noalloc_equals_workspace_call(woq, seq):
    lib = woq.load()
    cap = lib.woq_linear_noalloc_max_workspace_bytes()
    assert cap == 32 << 20
    for i, (m, n, k, group, with_order) in enumerate(seq):
        _say(f"noalloc call {i}: m={m} n={n} k={k} g={group} order={with_order} "
             f"plan: {woq.linear_plan(m, n, k, group, with_order)}")
        dev, ref = _case(woq, m, n, k, group, 9100 + 10 * i + m, with_order)
        for dt in (torch.float32, torch.bfloat16):
            y_na = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
            y_ws = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
            assert _noalloc(lib, dev, m, n, k, group, y_na) == 0
            st, need = _with_workspace(lib, dev, m, n, k, group, y_ws)
            assert st == 0 and need <= cap
            torch.cuda.synchronize()
            assert torch.equal(y_na, y_ws), f"call {i}: the two entry points differ"
            check_linear(y_na, ref, f"noalloc call {i} m={m} n={n} k={k}")


def test_noalloc_keeps_k_whole_when_the_partials_do_not_fit(woq, monkeypatch):
    """512 x 4096 x 4096 splits K in 4 with the caller's workspace (34 MB of
    partial outputs, more than the array); without allocating it runs the
    same tiles with K whole: bit-identical to the workspace call told to keep K
    whole, and within the gate of the oracle.  Then a smaller call."""
    lib = woq.load()
    cap = lib.woq_linear_noalloc_max_workspace_bytes()
    for i, (m, n, k, group, with_order) in enumerate([(512, 4096, 4096, 128, False), (40, 300, 1024, 64, True)]):
        monkeypatch.delenv("WOQ_GEMM_SPLITS", raising=False)
        plan = woq.linear_plan(m, n, k, group, with_order)
        _say(f"noalloc unsplit call {i}: m={m} n={n} k={k} g={group} plan: {plan}")
        if i == 0:
            assert "k_splits=4" in plan and lib.woq_linear_workspace_bytes(m, n, k, group, 0) > cap
        dev, ref = _case(woq, m, n, k, group, 9300 + 10 * i + m, with_order)
        for dt in (torch.float32, torch.bfloat16):
            y_na = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
            y_ws = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
            monkeypatch.delenv("WOQ_GEMM_SPLITS", raising=False)
            assert _noalloc(lib, dev, m, n, k, group, y_na) == 0
            # the reference call: the workspace entry point with K kept whole
            monkeypatch.setenv("WOQ_GEMM_SPLITS", "1")
            if i == 0:
                assert "k_splits=1" in woq.linear_plan(m, n, k, group, with_order)
            st, need = _with_workspace(lib, dev, m, n, k, group, y_ws)
            monkeypatch.delenv("WOQ_GEMM_SPLITS", raising=False)
            assert st == 0 and need <= cap
            torch.cuda.synchronize()
            assert torch.equal(y_na, y_ws), f"call {i}: the two entry points differ"
            check_linear(y_na, ref, f"noalloc unsplit call {i} m={m} n={n} k={k}")


def test_noalloc_refuses_sizes_beyond_its_array(woq):
    lib = woq.load()
    _say("noalloc size limit")
    m, n, k, group = 2048, 4096, 14336, 128
    need = lib.woq_linear_workspace_bytes(m, n, k, group, 0)
    assert need > lib.woq_linear_noalloc_max_workspace_bytes()
    one = torch.zeros(16, dtype=torch.uint8, device="cuda")
    y = torch.zeros(16, dtype=torch.float32, device="cuda")
    st = lib.woq_linear_int4_groups_noalloc(one.data_ptr(), m, one.data_ptr(), one.data_ptr(), one.data_ptr(),
                                            None, None, n, k, group, 0, y.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream)
    assert woq.STATUS[st] == "WOQ_EWORKSPACE"
    # no workspace needed: m == 0 and decode without a gather run as the plain call
    assert lib.woq_linear_int4_groups_noalloc(None, 0, None, None, None, None, None, n, k, group, 0, None,
                                              None) == 0
