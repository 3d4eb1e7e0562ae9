"""Pins for the oracle's AWQ scale search (R14).

"20. Quantization" (inference book), stretch exercise 3: for one linear layer,
search a per-input-channel scale s_j = mean|x_j|^alpha over alpha in [0, 1]
for the least calibration output error after 4-bit quantization of
W diag(s); the scaling identity X W^T = (X S^-1)(W S)^T of the same page says
the scaled layer computes with X S^-1.  The grid, the floor and the tie rule
are the readings the oracle states (R14).

The pins: a tiny case whose scales are powers of two, brute-forced in exact
rational arithmetic over a three-point grid; channels of equal magnitude,
where every alpha gives the same layer and the search returns round to
nearest; a salient channel, whose protection lowers the error, with the
alpha = 0 point equal to round to nearest's output error; a dead channel at
the floor; and the chosen error equal to the directly computed error of the
layer (X S^-1) dequant^T.
"""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest

import oracle


def oracle_impl():
    return SimpleNamespace(awq=oracle.awq_search)


def check_tiny_brute_force(impl):
    # mean |x_j| = 4, 1, 1/4, 1/16 with signs mixed so that the signed means are 0
    x = np.array([[4, 1, 0.25, 0.0625],
                  [-4, -1, -0.25, 0.0625],
                  [4, -1, 0.25, -0.0625],
                  [-4, 1, -0.25, -0.0625]], dtype=np.float32)
    w = np.array([[0.3, -0.7, 0.11, 0.9], [-0.25, 0.05, 0.6, -0.45]], dtype=np.float32)
    q, sc, z, s, best, losses = impl.awq(w, x, 2, n_grid=2)
    assert len(losses) == 3
    exact = []
    for i, sj in enumerate(([1, 1, 1, 1], [2, 1, 0.5, 0.25], [4, 1, 0.25, 0.0625])):
        s_i = np.array(sj, np.float32)
        ws = w * s_i                                        # powers of two: exact in float32
        qi, sci, zi = oracle.quantize_groups(ws, 2)
        err = Fraction(0)
        for t in range(4):
            for r in range(2):
                acc = Fraction(0)
                for c in range(4):
                    w_hat = (int(qi[r, c]) - int(zi[r, c // 2])) * Fraction(float(sci[r, c // 2])) / Fraction(sj[c])
                    acc += Fraction(float(x[t, c])) * (Fraction(float(w[r, c])) - w_hat)
                err += acc * acc
        exact.append(err)
        assert abs(losses[i] - float(err)) <= 1e-12 * float(err), (i, losses[i], float(err))
        if i == best:
            assert np.array_equal(s, s_i) and np.array_equal(q, qi) and np.array_equal(sc, sci) and np.array_equal(z, zi)
    assert best == min(range(3), key=lambda i: (exact[i], i))


def check_equal_channels_is_rtn(impl):
    rng = np.random.default_rng(13)
    x = np.where(rng.random((16, 64)) < 0.5, -1.0, 1.0).astype(np.float32)   # mean |x_j| = 1 everywhere
    w = (rng.standard_normal((8, 64)) * 0.05).astype(np.float32)
    q, sc, z, s, best, losses = impl.awq(w, x, 16)
    assert best == 0 and np.all(losses == losses[0])
    assert np.all(s == 1)
    qr, sr, zr = oracle.quantize_groups(w, 16)
    assert np.array_equal(q, qr) and np.array_equal(sc, sr) and np.array_equal(z, zr)


def _salient_case(seed=17, n=16, k=64):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((48, k))
    x[:, 3] *= 30.0
    x[:, 40] *= 12.0
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    return w, x.astype(np.float32)


def check_salient_channel_protected(impl):
    w, x = _salient_case()
    n, k = w.shape
    q, sc, z, s, best, losses = impl.awq(w, x, 16)
    assert best > 0 and losses[best] < 0.5 * losses[0]
    assert s[3] > np.max(np.delete(s, [3, 40]))
    # alpha = 0 is round to nearest
    qr, sr, zr = oracle.quantize_groups(w, 16)
    w_rtn = oracle.dequantize_int4_groups(oracle.pack_uint4(qr), sr, zr, n, k, 16).astype(np.float64)
    e = x.astype(np.float64) @ (w.astype(np.float64) - w_rtn).T
    assert abs(losses[0] - np.sum(e * e)) <= 1e-6 * losses[0]


def check_dead_channel_floor(impl):
    w, x = _salient_case(seed=19)
    x[:, 9] = 0.0
    q, sc, z, s, best, losses = impl.awq(w, x, 16)
    assert best > 0
    assert s[9] == np.float32(1e-4)


def check_error_is_the_scaled_layers(impl):
    w, x = _salient_case(seed=23, n=24, k=128)
    n, k = w.shape
    q, sc, z, s, best, losses = impl.awq(w, x, 32)
    deq = oracle.dequantize_int4_groups(oracle.pack_uint4(q), sc, z, n, k, 32).astype(np.float64)
    y = x.astype(np.float64) @ w.astype(np.float64).T
    y_hat = (x.astype(np.float64) / s.astype(np.float64)) @ deq.T
    assert abs(np.sum((y - y_hat) ** 2) - losses[best]) <= 1e-6 * losses[best]
    assert losses[best] == np.min(losses)


ALL_CHECKS = [check_tiny_brute_force, check_equal_channels_is_rtn, check_salient_channel_protected,
              check_dead_channel_floor, check_error_is_the_scaled_layers]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle_impl())


# ---------------------------------------------------------------------------
# Planted mistakes: test-only copies of the search with one deviation each
# ---------------------------------------------------------------------------

def _awq_variant(w, x, group, n_grid=20, signed=False, power=1.0, unscale=True, worst=False, with_end=True,
                 floor_first=False):
    w = np.asarray(w, np.float32)
    n, k = w.shape
    xv = np.asarray(x, np.float64)
    m = xv.mean(axis=0) if signed else np.abs(xv).mean(axis=0)
    losses, best = [], None
    for i in range(n_grid + 1 if with_end else n_grid):
        a = power * i / n_grid
        if floor_first:
            s = np.power(np.maximum(m, oracle.AWQ_FLOOR), a).astype(np.float32)
        else:
            s = np.maximum(np.power(m, a), oracle.AWQ_FLOOR).astype(np.float32)
        ws = (w.astype(np.float64) * s).astype(np.float32)
        q, sc, zr = oracle.quantize_groups(ws, group)
        deq = ((q.reshape(n, k // group, group).astype(np.float64) - zr[:, :, None]) * sc[:, :, None]).reshape(n, k)
        w_hat = deq / s if unscale else deq
        e = xv @ (w.astype(np.float64) - w_hat).T
        losses.append(float(np.sum(e * e)))
        better = best is None or (losses[-1] > losses[best[0]] if worst else losses[-1] < losses[best[0]])
        if better:
            best = (i, q, sc, zr, s)
    i, q, sc, zr, s = best
    return q, sc, zr, s, i, np.array(losses)


def _mutant(**kw):
    return SimpleNamespace(awq=lambda *a, **k2: _awq_variant(*a, **k2, **kw))


MUTANTS = {
    "signed_mean": lambda: _mutant(signed=True),
    "inverse_power": lambda: _mutant(power=-1.0),
    "activations_not_unscaled": lambda: _mutant(unscale=False),
    "largest_error_chosen": lambda: _mutant(worst=True),
    "grid_without_alpha_one": lambda: _mutant(with_end=False),
    "floor_before_power": lambda: _mutant(floor_first=True),
}


def test_variant_without_mistakes_passes():
    for check in ALL_CHECKS:
        check(_mutant())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    impl = MUTANTS[name]()
    caught = []
    for check in ALL_CHECKS:
        try:
            check(impl)
        except (AssertionError, ValueError, IndexError, pytest.fail.Exception) as exc:
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"planted mistake {name} passed every check"
