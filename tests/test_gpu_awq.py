"""GPU AWQ scale search against the float64 oracle.

"20. Quantization" (inference book), stretch exercise 3, with the grid, floor
and tie rule the oracle states.  Both sides take every decision that makes an
integer from the same float64 or float32 values: the scales (float32 of a
float64 power), the scaled weights (a float32 product), the group quantizer
(its float64 rule).  The errors of the grid points are float64 sums in
different orders, equal to about 1e-13 relative; the chosen point must be the
oracle's (or, where two points' errors lie within 1e-9 of each other, one the
oracle rates as low), and at the chosen point the scales, codes, scales and
zeros are bit-identical.  Each case prints its name first.
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
    q, sc, z, s, best, losses = got
    qr, scr, zr, sr, best_r, losses_r = want
    losses = losses.cpu().numpy()
    assert losses.shape == losses_r.shape, what
    assert np.allclose(losses, losses_r, rtol=1e-9, atol=0), f"{what}: errors {losses} vs {losses_r}"
    if best != best_r:
        assert losses_r[best] <= losses_r[best_r] * (1 + 1e-9), f"{what}: chose {best}, oracle {best_r}"
        return
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32)), f"{what}: s"
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), scr.view(np.uint32)), f"{what}: scale"
    assert np.array_equal(z.cpu().numpy(), zr), f"{what}: zero"
    bad = np.argwhere(q.cpu().numpy() != qr)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[:4].tolist()}"


CASES = [
    # n, k, t, group, n_grid, channel spread, dead channels
    (16, 64, 48, 16, 20, 1.5, ()),
    (24, 128, 48, 32, 20, 1.5, (9,)),
    (70, 192, 100, 64, 20, 1.0, ()),       # ragged tiles in both directions
    (5, 40, 3, 8, 4, 1.0, ()),
    (33, 256, 130, 128, 20, 0.5, ()),
    (130, 512, 64, 256, 10, 1.0, (0, 511)),
]


@pytest.mark.parametrize("n,k,t,group,n_grid,spread,dead", CASES)
def test_awq_matches_oracle(woq, n, k, t, group, n_grid, spread, dead):
    _say(f"awq n={n} k={k} t={t} group={group} n_grid={n_grid} spread={spread} dead={dead}")
    w = workloads.weight(n, k, seed=n + 2 * k)
    x = workloads.calibration_bf16(t, k, seed=t + 3 * k, channel_spread=spread)
    for c in dead:
        x[:, c] = 0
    got = woq.awq_search(torch.from_numpy(w).cuda(), to_dev_bf16(x), group, n_grid=n_grid)
    torch.cuda.synchronize()
    _compare(got, oracle.awq_search(w, x, group, n_grid=n_grid), f"n={n} k={k}")
    if dead and got[4] > 0:
        assert all(got[3][c].item() == np.float32(1e-4) for c in dead)


def test_awq_errors(woq):
    _say("awq errors")
    w = torch.from_numpy(workloads.weight(8, 64, seed=1)).cuda()
    x = to_dev_bf16(workloads.calibration_bf16(16, 64, seed=2))
    bad = w.clone()
    bad[2, 3] = float("nan")
    with pytest.raises(woq_mod.WoqError) as e:
        woq.awq_search(bad, x, 16)
    assert e.value.status == 4
    with pytest.raises(woq_mod.WoqError) as e:
        woq.awq_search(w, x, 24)
    assert e.value.status == 3


@pytest.mark.slow
def test_awq_full_size_sampled(woq):
    n, k, t, group = 4096, 4096, 256, 128
    _say(f"awq full size n={n} k={k} t={t} group={group}")
    w = workloads.weight(n, k, seed=31)
    x = workloads.calibration_bf16(t, k, seed=32)
    wd, xd = torch.from_numpy(w).cuda(), to_dev_bf16(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    q, sc, z, s, best, losses = woq.awq_search(wd, xd, group)
    torch.cuda.synchronize()
    _say(f"  gpu awq {time.perf_counter() - t0:.3f} s, best alpha index {best}")
    losses = losses.cpu().numpy()
    assert best == int(np.argmin(losses))
    mean_abs = np.abs(oracle.bf16_bits_to_f64(x)).mean(axis=0)
    s_ref = oracle.awq_scales(mean_abs, best / 20)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    xv = oracle.bf16_bits_to_f64(x)
    for i in sorted({0, max(best - 1, 0), best, min(best + 1, 20), 20}):
        ref, *_ = oracle.awq_error(w, xv, group, oracle.awq_scales(mean_abs, i / 20))
        assert abs(losses[i] - ref) <= 1e-9 * ref, (i, losses[i], ref)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(6).choice(n, 30, replace=False)]))
    ws = (w[rows].astype(np.float64) * s_ref.astype(np.float64)).astype(np.float32)
    qr, scr, zr = oracle.quantize_groups(ws, group)
    ri = torch.from_numpy(rows).cuda()
    assert np.array_equal(q[ri].cpu().numpy(), qr)
    assert np.array_equal(sc[ri].cpu().numpy().view(np.uint32), scr.view(np.uint32))
    assert np.array_equal(z[ri].cpu().numpy(), zr)
