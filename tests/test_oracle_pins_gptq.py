"""Pins for the oracle's GPTQ (R13).

"20. Quantization" (inference book), stretch exercise 4: H = 2 X^T X from
calibration inputs, quantize column by column, spreading each column's error
over the remaining columns with the Cholesky factor of H^-1, compared with
round to nearest; linnet "Importing GPTQ and AWQ": activation order gives the
layer an `order` it gathers its inputs through.  The published method (Frantar
et al.) fixes the remaining steps: dead columns, ordering by decreasing H_jj,
damping, group parameters taken when a group starts.

The pins: where H is diagonal the method reduces to round to nearest; the
update of a column by one earlier column has the closed form
w_j += (w_i - dequant_i) * H_ij / H_jj (the optimal-brain-surgeon step) when
only those two columns are coupled; a later group's parameters come from its
updated columns; the visiting order is the stable sort of H_jj, decreasing; and
on correlated calibration data the output error falls below round to nearest.
"""
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
import workloads


def oracle_impl():
    return SimpleNamespace(gptq=oracle.gptq_quantize)


def _rtn_code(w, scale, zero):
    """R2 code of real values w against a group's (scale, zero), exact arithmetic."""
    from fractions import Fraction
    rng_ = Fraction(float(scale)) * 15
    out = []
    for v in np.atleast_1d(w):
        t = Fraction(float(v)) * 15 / rng_
        out.append(int(min(15, max(0, round(t) + int(zero)))))
    return out


def _dequant(q, s, z, n, k, g):
    return oracle.dequantize_int4_groups(oracle.pack_uint4(q), s, z, n, k, g).astype(np.float64)


def check_diagonal_h_is_round_to_nearest(impl):
    rng = np.random.default_rng(3)
    k, group = 64, 16
    w = (rng.standard_normal((8, k)) * 0.02).astype(np.float32)
    x = np.diag(rng.uniform(0.5, 2.0, size=k)).astype(np.float32)     # orthogonal columns: H diagonal
    q, s, z, order = impl.gptq(w, x, group)
    qr, sr, zr = oracle.quantize_groups(w, group)
    assert order is None
    assert np.array_equal(q, qr) and np.array_equal(s, sr) and np.array_equal(z, zr)
    q, s, z, order = impl.gptq(w, x, group, act_order=True)
    d2 = np.diag(x.astype(np.float64)) ** 2
    assert np.array_equal(order, np.argsort(-d2, kind="stable"))
    qr, sr, zr = oracle.quantize_groups(w[:, order], group)
    assert np.array_equal(q, qr) and np.array_equal(s, sr) and np.array_equal(z, zr)


def check_two_column_update_closed_form(impl):
    # one group of two columns; H = [[a, b], [b, c]] (+ damping); column 0 is
    # coded, then column 1 becomes w1 + (w0 - dq0) * H01 / H11 and is coded
    # with the group's parameters
    x = np.array([[1.0, 0.9], [0.3, 1.0], [0.5, -0.2], [1.0, 1.0]], dtype=np.float32)
    damp = 0.01
    h = x.astype(np.float64).T @ x.astype(np.float64)
    h = h + damp * np.mean(np.diag(h)) * np.eye(2)
    for w0, w1 in ((0.37, -0.81), (1.13, 0.05), (-0.6, 0.61)):
        w = np.array([[w0, w1]], dtype=np.float32)
        q, s, z, _ = impl.gptq(w, x, 2, damp=damp)
        # the group parameters are those of the original pair (taken before any update)
        qr, sr, zr = oracle.quantize_groups(w, 2)
        assert s[0, 0] == sr[0, 0] and z[0, 0] == zr[0, 0]
        assert q[0, 0] == qr[0, 0]
        dq0 = (int(qr[0, 0]) - int(zr[0, 0])) * float(sr[0, 0])
        w1_new = float(w1) + (float(w0) - dq0) * h[0, 1] / h[1, 1]
        assert q[0, 1] == _rtn_code([w1_new], sr[0, 0], zr[0, 0])[0], (w0, w1, w1_new)


def check_later_group_takes_updated_columns(impl):
    # columns 0 and 2 coupled only; groups {0, 1} and {2, 3}: group 1's range comes
    # from w2 + (w0 - dq0) * H02 / H22 and w3
    x = np.zeros((8, 4), np.float32)
    x[:5, 0] = [1.0, 0.5, -0.3, 0.8, 0.1]
    x[:5, 2] = [0.9, 0.6, -0.1, 0.7, -0.4]
    x[6, 1] = 1.0                                       # columns 1 and 3 each on a row of their own
    x[7, 3] = 0.5
    h = x.astype(np.float64).T @ x.astype(np.float64)
    assert h[0, 1] == 0 and h[0, 3] == 0 and h[1, 2] == 0 and h[2, 3] == 0 and h[1, 3] == 0
    damp = 0.01
    hd = h + damp * np.mean(np.diag(h)) * np.eye(4)
    w = np.array([[0.9, -0.2, 0.1, -0.3]], dtype=np.float32)
    q, s, z, _ = impl.gptq(w, x, 2, damp=damp)
    qr, sr, zr = oracle.quantize_groups(w[:, :2], 2)
    dq0 = (int(qr[0, 0]) - int(zr[0, 0])) * float(sr[0, 0])
    w2_new = float(w[0, 2]) + (float(w[0, 0]) - dq0) * hd[0, 2] / hd[2, 2]
    lo, hi = min(w2_new, float(w[0, 3])), max(w2_new, float(w[0, 3]))
    assert s[0, 1] == np.float32((hi - lo) / 15)
    assert s[0, 1] != oracle.quantize_groups(w[:, 2:], 2)[1][0, 0]     # not the original pair's


def check_order_is_a_stable_decreasing_sort(impl):
    rng = np.random.default_rng(5)
    k = 32
    x = rng.standard_normal((64, k)).astype(np.float32)
    x[:, 7] = x[:, 3]                                   # equal H_jj: the earlier column first
    w = (rng.standard_normal((4, k)) * 0.02).astype(np.float32)
    _, _, _, order = impl.gptq(w, x, 16, act_order=True)
    d = np.diag(x.astype(np.float64).T @ x.astype(np.float64))
    assert sorted(order.tolist()) == list(range(k))
    assert np.all(np.diff(d[order]) <= 0)
    assert order.tolist().index(3) < order.tolist().index(7)


def check_dead_column_is_zero(impl):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((32, 16)).astype(np.float32)
    x[:, 5] = 0.0
    w = (rng.standard_normal((3, 16)) * 0.1).astype(np.float32)
    q, s, z, _ = impl.gptq(w, x, 16)
    wd = _dequant(q, s, z, 3, 16, 16)
    assert np.all(np.abs(wd[:, 5]) <= s[:, 0].astype(np.float64) / 2)   # the weight became 0: its nearest level


def check_beats_round_to_nearest(impl):
    rng = np.random.default_rng(11)
    n, k, t = 32, 128, 512
    base = rng.standard_normal((t, 16))
    x = (base @ rng.standard_normal((16, k)) + 0.3 * rng.standard_normal((t, k))).astype(np.float32)
    for group, act_order in ((32, False), (128, True)):
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        q, s, z, order = impl.gptq(w, x, group, act_order=act_order)
        xo = x if order is None else x[:, order]
        y = x.astype(np.float64) @ w.T.astype(np.float64)
        e_gptq = np.linalg.norm(y - xo.astype(np.float64) @ _dequant(q, s, z, n, k, group).T)
        qr, sr, zr = oracle.quantize_groups(w, group)
        e_rtn = np.linalg.norm(y - x.astype(np.float64) @ _dequant(qr, sr, zr, n, k, group).T)
        assert e_gptq < 0.8 * e_rtn, (group, act_order, e_gptq, e_rtn)


ALL_CHECKS = [check_diagonal_h_is_round_to_nearest, check_two_column_update_closed_form,
              check_later_group_takes_updated_columns, check_order_is_a_stable_decreasing_sort,
              check_dead_column_is_zero, check_beats_round_to_nearest]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle_impl())


# ---------------------------------------------------------------------------
# Planted mistakes: test-only copies of the sweep with one deviation each
# ---------------------------------------------------------------------------

def _gptq_variant(w, x, group, act_order=False, damp=0.01, propagate=1.0, params_from_original=False,
                  ascending=False):
    w = np.asarray(w, np.float32)
    n, k = w.shape
    xv = np.asarray(x, np.float64)
    W = w.astype(np.float64)
    H = xv.T @ xv
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    W[:, dead] = 0.0
    perm = None
    if act_order:
        perm = np.argsort(np.diag(H) if ascending else -np.diag(H), kind="stable")
        W, H = W[:, perm], H[perm][:, perm]
    W0 = W.copy()
    H = H + damp * np.mean(np.diag(H)) * np.eye(k)
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    q = np.zeros((n, k), np.uint8)
    scale = np.zeros((n, k // group), np.float32)
    zero = np.zeros((n, k // group), np.uint8)
    for i in range(k):
        g = i // group
        if i % group == 0:
            src = W0 if params_from_original else W
            sc, zr, flat, d_safe = oracle.woq_ref._asym_group_params(src[:, i:i + group])
            scale[:, g], zero[:, g] = sc, zr
        col = W[:, i]
        r = np.where(flat, np.rint(col), np.rint(15 * col / d_safe))
        qi = np.clip(r + zero[:, g], 0, 15)
        q[:, i] = qi
        err = (col - (qi - zero[:, g].astype(np.float64)) * scale[:, g].astype(np.float64)) / U[i, i]
        W[:, i + 1:] -= propagate * np.outer(err, U[i, i + 1:])
    return q, scale, zero, (None if perm is None else perm.astype(np.int32))


MUTANTS = {
    "no_error_propagation": lambda: SimpleNamespace(gptq=lambda *a, **kw: _gptq_variant(*a, propagate=0.0, **kw)),
    "propagation_sign_flipped": lambda: SimpleNamespace(gptq=lambda *a, **kw: _gptq_variant(*a, propagate=-1.0, **kw)),
    "group_params_from_original_weights": lambda: SimpleNamespace(
        gptq=lambda *a, **kw: _gptq_variant(*a, params_from_original=True, **kw)),
    "order_ascending": lambda: SimpleNamespace(gptq=lambda *a, **kw: _gptq_variant(*a, ascending=True, **kw)),
}


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


def test_gptq_refuses_a_singular_undamped_matrix():
    """Without damping, two equal input channels orthogonal to the rest make H
    exactly singular: the inverse the method factors does not exist, and the
    oracle raises instead of returning codes from a meaningless factor."""
    n, k, t, group = 4, 32, 8, 16
    w = workloads.weight(n, k, seed=43)
    x = workloads.calibration_bf16(t, k, seed=44)
    x[:, :2] = 0
    x[0, :] = 0
    x[0, :2] = 0x4000
    with pytest.raises(np.linalg.LinAlgError):
        oracle.gptq_quantize(w, x, group, damp=0.0)
    q, s, z, _ = oracle.gptq_quantize(w, x, group, damp=0.01)
    assert q.shape == (n, k) and np.all(np.isfinite(s))
