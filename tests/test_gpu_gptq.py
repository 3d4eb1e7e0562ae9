"""GPU GPTQ against the float64 oracle.

"20. Quantization" (inference book), stretch exercise 4, with the steps the
published method fixes (dead columns, activation order, damping, group
parameters when a group starts); linnet "Importing GPTQ and AWQ" for the
`order` the layer gathers through.  Both sides decide every code in float64;
the only difference is the rounding of the factorization of H (the oracle
inverts and factors with LAPACK, the kernels factor the reversed H and invert
the triangle), about 1e-13 relative, so a code could differ only where a
quotient lands that close to a rounding tie: the codes, scales, zeros and
order are required to be equal.  Rows are independent given H, so at full
size the oracle quantizes a sample of rows.  Each case prints its name first.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import workloads
import weight_only_quantization_amd as woq_mod
from helpers import to_dev_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _compare(got, want, what):
    q, s, z, o = (None if v is None else v.cpu().numpy() for v in got)
    qr, sr, zr, orr = want
    assert (o is None) == (orr is None), what
    if o is not None:
        assert np.array_equal(o, orr), f"{what}: order"
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), f"{what}: scale"
    assert np.array_equal(z, zr), f"{what}: zero"
    bad = np.argwhere(q != qr)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[:4].tolist()}"


CASES = [
    # n, k, t, group, act_order, dead columns
    (32, 128, 256, 32, False, ()),
    (48, 384, 512, 128, True, ()),
    (70, 288, 300, 96, True, (5, 200)),     # blocks of 192 columns: one whole, one of 96
    (33, 512, 100, 256, False, ()),
    (5, 130, 64, 2, True, (0,)),            # a ragged last block of 2 columns
    (4, 129, 40, 3, False, ()),             # odd K, blocks of 129
    (65, 256, 0, 64, True, ()),             # no calibration rows: every column dead
]


@pytest.mark.parametrize("n,k,t,group,act_order,dead", CASES)
def test_gptq_matches_oracle(woq, n, k, t, group, act_order, dead):
    _say(f"gptq n={n} k={k} t={t} group={group} act_order={act_order} dead={dead}")
    w = workloads.weight(n, k, seed=n + k)
    x = workloads.calibration_bf16(max(t, 1), k, seed=t + k)[:t]
    for c in dead:
        x[:, c] = 0
    got = woq.gptq_quantize(torch.from_numpy(w).cuda(), to_dev_bf16(x) if t else None, group,
                            act_order=act_order)
    torch.cuda.synchronize()
    _compare(got, oracle.gptq_quantize(w, x if t else np.zeros((0, k), np.uint16), group, act_order=act_order),
             f"n={n} k={k}")


def test_gptq_diagonal_h_is_group_rtn(woq):
    _say("gptq diagonal H")
    n, k, group = 40, 256, 64
    w = workloads.weight(n, k, seed=3)
    d = workloads.calibration_bf16(1, k, seed=4)[0]
    d[(d & 0x7FFF) == 0] = 0x3F80                      # no dead column: a zero becomes 1.0
    x = np.zeros((k, k), np.uint16)
    x[np.arange(k), np.arange(k)] = d                  # orthogonal input channels: H diagonal
    q, s, z, o = woq.gptq_quantize(torch.from_numpy(w).cuda(), to_dev_bf16(x), group)
    qr, sr, zr = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
    torch.cuda.synchronize()
    assert o is None
    assert torch.equal(q, qr) and torch.equal(s, sr) and torch.equal(z, zr)


def test_gptq_damping_and_errors(woq):
    _say("gptq damping and errors")
    n, k, group = 16, 128, 32
    w = workloads.weight(n, k, seed=8)
    x = workloads.calibration_bf16(64, k, seed=9)
    got = woq.gptq_quantize(torch.from_numpy(w).cuda(), to_dev_bf16(x), group, damp=0.1)
    torch.cuda.synchronize()
    _compare(got, oracle.gptq_quantize(w, x, group, damp=0.1), "damp=0.1")
    bad = torch.from_numpy(w).cuda()
    bad[3, 7] = float("inf")
    with pytest.raises(woq_mod.WoqError) as e:
        woq.gptq_quantize(bad, to_dev_bf16(x), group)
    assert e.value.status == 4


@pytest.mark.slow
@pytest.mark.parametrize("act_order", [False, True])
def test_gptq_full_size_sampled(woq, act_order):
    n, k, t, group = 4096, 4096, 256, 128
    _say(f"gptq full size n={n} k={k} t={t} group={group} act_order={act_order}")
    w = workloads.weight(n, k, seed=21)
    x = workloads.calibration_bf16(t, k, seed=22)
    wd, xd = torch.from_numpy(w).cuda(), to_dev_bf16(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got = woq.gptq_quantize(wd, xd, group, act_order=act_order)
    torch.cuda.synchronize()
    _say(f"  gpu gptq {time.perf_counter() - t0:.3f} s")
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(5).choice(n, 14, replace=False)]))
    q, s, z, o = got
    sub = (q[torch.from_numpy(rows).cuda()], s[torch.from_numpy(rows).cuda()], z[torch.from_numpy(rows).cuda()], o)
    _compare(sub, oracle.gptq_quantize(w[rows], x, group, act_order=act_order), f"full act_order={act_order}")


def _singular_calibration(t, k, seed):
    """Inputs 0 and 1 equal (2.0 in row 0 only) and orthogonal to every other
    input: H has the 2x2 block [[4, 4], [4, 4]] apart from the rest, so with no
    damping the factorization meets an exactly zero pivot in any column order."""
    x = workloads.calibration_bf16(t, k, seed=seed)
    x[:, :2] = 0
    x[0, :] = 0
    x[0, :2] = 0x4000                                   # bf16 2.0
    return x


def test_gptq_not_positive_definite(woq):
    _say("gptq singular calibration matrix, no damping")
    n, k, t, group = 8, 64, 16, 32
    w = workloads.weight(n, k, seed=41)
    x = _singular_calibration(t, k, 42)
    with pytest.raises(np.linalg.LinAlgError):
        oracle.gptq_quantize(w, x, group, damp=0.0)
    for act_order in (False, True):
        with pytest.raises(woq_mod.WoqError) as e:
            woq.gptq_quantize(torch.from_numpy(w).cuda(), to_dev_bf16(x), group, act_order=act_order, damp=0.0)
        assert e.value.name == "WOQ_ENOTPD"
    # the same inputs with damping factor fine on both sides
    got = woq.gptq_quantize(torch.from_numpy(w).cuda(), to_dev_bf16(x), group, damp=0.01)
    torch.cuda.synchronize()
    _compare(got, oracle.gptq_quantize(w, x, group, damp=0.01), "singular x, damp=0.01")


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("act_order", [False, True])
def test_gptq_long_rows_sampled(woq, act_order):
    """K = 14336 (the down projection's input width): 448 panels of the
    blocked factorization; codes, scales, zeros and order of sampled rows equal
    to the oracle's."""
    n, k, t, group = 4096, 14336, 256, 128
    _say(f"gptq long rows n={n} k={k} t={t} group={group} act_order={act_order}")
    w = workloads.weight(n, k, seed=61)
    x = workloads.calibration_bf16(t, k, seed=62)
    wd, xd = torch.from_numpy(w).cuda(), to_dev_bf16(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got = woq.gptq_quantize(wd, xd, group, act_order=act_order)
    torch.cuda.synchronize()
    _say(f"  gpu gptq {time.perf_counter() - t0:.3f} s")
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(7).choice(n, 6, replace=False)]))
    q, s, z, o = got
    idx = torch.from_numpy(rows).cuda()
    t0 = time.perf_counter()
    want = oracle.gptq_quantize(w[rows], x, group, act_order=act_order)
    _say(f"  oracle gptq on {len(rows)} rows {time.perf_counter() - t0:.1f} s")
    _compare((q[idx], s[idx], z[idx], o), want, f"long rows act_order={act_order}")
