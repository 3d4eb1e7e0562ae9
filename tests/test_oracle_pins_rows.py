"""Pins for the oracle's Int4Linear functions (R12): signed int4, one float32 scale a row.

linnet docs "Quantization" (std.quant table: Int4Linear weight [Out, In/2] of
signed nibbles, even element in the low nibble; one float32 scale a row as the
page's Mlp example declares; dequantize_int4 = unpack, then dequantize) and
tinyllm L8.5 section 2 (symmetric scaling s = amax / q_max, codes rint(W / s)
with quotients formed in float32, a zero row gets s = 0 and codes 0) with
q_max = 7, and its section 3 worked example, whose rows are one group each.

Each check takes an implementation namespace; the oracle must pass every
check and each planted mistake must fail at least one.
"""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from conftest import load_golden, parse_nums


def _nearest_f32(fr: Fraction) -> Fraction:
    c = np.float32(float(fr))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = None
    for cand in sorted(cands):
        key = (abs(Fraction(float(cand)) - fr), int(np.array(cand, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return Fraction(float(best[1]))


def _expect_row(wrow):
    amax = max((abs(Fraction(float(v))) for v in wrow), default=Fraction(0))
    s = _nearest_f32(amax / 7)
    if s == 0:
        return [0] * len(wrow), 0.0
    codes = [max(-8, min(7, round(_nearest_f32(Fraction(float(v)) / s)))) for v in wrow]
    return codes, float(s)


def oracle_impl():
    return SimpleNamespace(quantize=oracle.quantize_int4_rows, pack=oracle.pack_int4,
                           dequantize=oracle.dequantize_int4_rows, linear=oracle.linear_int4_rows)


def check_worked_example(impl):
    g = load_golden("symmetric_int4_group4_rows.txt")
    w = np.array([[float(v) for v in parse_nums(g["row0_w"])],
                  [float(v) for v in parse_nums(g["row1_w"])]], dtype=np.float32)
    c, s = impl.quantize(w)
    assert np.asarray(c).tolist() == [[int(v) for v in parse_nums(g["row0_codes"])],
                                      [int(v) for v in parse_nums(g["row1_codes"])]]
    assert np.asarray(s).dtype == np.float32 and np.asarray(s).tolist() == [0.25, 0.25]
    packed = impl.pack(c)
    assert np.asarray(packed).tolist() == [[int(v, 16) for v in g["row0_bytes_hex"].split()],
                                           [int(v, 16) for v in g["row1_bytes_hex"].split()]]
    w_hat = impl.dequantize(packed, s, 2, 4)
    assert w_hat.tolist() == [[float(v) for v in parse_nums(g["row0_w_hat"])],
                              [float(v) for v in parse_nums(g["row1_w_hat"])]]


def check_bruteforce(impl):
    rng = np.random.default_rng(29)
    for trial in range(30):
        k = [2, 6, 16, 40][trial % 4]
        w = (rng.standard_normal((3, k)) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        if trial % 5 == 0:
            w[1] = 0.0
        c, s = impl.quantize(w)
        for r in range(3):
            codes, sr = _expect_row(w[r])
            assert float(np.asarray(s)[r]) == sr, (trial, r)
            assert np.asarray(c)[r].tolist() == codes, (trial, r)


def check_zero_row_and_refusals(impl):
    c, s = impl.quantize(np.zeros((2, 8), np.float32))
    assert np.all(np.asarray(c) == 0) and np.all(np.asarray(s) == 0)
    assert np.all(impl.dequantize(impl.pack(c), s, 2, 8) == 0)
    for bad in (np.array([[0.0, np.nan]], np.float32), np.ones((2, 3), np.float32), np.ones(4, np.float32)):
        with pytest.raises(ValueError):
            impl.quantize(bad)


def check_half_step(impl):
    rng = np.random.default_rng(31)
    for log_s in np.linspace(-3, 2, 11):
        w = (rng.standard_normal((8, 96)) * 10.0 ** log_s).astype(np.float32)
        c, s = impl.quantize(w)
        s64 = np.asarray(s, np.float64)[:, None]
        err = np.abs(np.asarray(c, np.float64) * s64 - w.astype(np.float64))
        assert np.all(err <= s64 / 2 * (1 + 2.0 ** -20))


def check_dequant_rounding(impl):
    rng = np.random.default_rng(37)
    n, k = 5, 24
    c = rng.integers(-8, 8, size=(n, k)).astype(np.int8)
    s = rng.uniform(0.001, 3.0, size=n).astype(np.float32)
    got = impl.dequantize(impl.pack(c), s, n, k)
    for r in range(n):
        for j in range(k):
            assert Fraction(float(got[r, j])) == _nearest_f32(int(c[r, j]) * Fraction(float(s[r])))


def check_linear_exact(impl):
    rng = np.random.default_rng(41)
    for m, n, k, with_bias, with_order in ((1, 3, 8, False, False), (2, 4, 16, True, True)):
        c = rng.integers(-8, 8, size=(n, k)).astype(np.int8)
        s = rng.uniform(0.01, 2.0, size=n).astype(np.float32)
        x = rng.standard_normal((m, k)).astype(np.float32)
        bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
        order = rng.permutation(k).astype(np.int32) if with_order else None
        y = impl.linear(x, impl.pack(c), s, n, k, bias=bias, order=order)
        xs = x[:, order] if order is not None else x
        for i in range(m):
            for j in range(n):
                acc = sum(Fraction(float(xs[i, t])) * int(c[j, t]) * Fraction(float(s[j])) for t in range(k))
                if bias is not None:
                    acc += Fraction(float(bias[j]))
                assert abs(y[i, j] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))


ALL_CHECKS = [check_worked_example, check_bruteforce, check_zero_row_and_refusals, check_half_step,
              check_dequant_rounding, check_linear_exact]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle_impl())


def _quantize_variant(w, qmax=7, zero_scale=0.0, rnd=np.rint, f64_scale=False):
    w = np.asarray(w, np.float32)
    if w.ndim != 2 or w.shape[1] % 2 or not np.all(np.isfinite(w)):
        raise ValueError("bad")
    amax = np.abs(w).max(1)
    s = (amax.astype(np.float64) / qmax) if f64_scale else (amax / np.float32(qmax)).astype(np.float32)
    live = s > 0
    c = np.clip(rnd(w / np.where(live, s, 1)[:, None]), -8, 7)
    c = np.where(live[:, None], c, 0)
    s = np.where(live, s, zero_scale).astype(np.float32)
    return c.astype(np.int8), s


def _pack_swapped(c):
    c = np.asarray(c)
    if c.shape[-1] % 2:
        raise ValueError("bad")
    sw = c.copy()
    sw[..., 0::2], sw[..., 1::2] = c[..., 1::2], c[..., 0::2]
    return oracle.pack_int4(sw)


def _linear_no_bias(x, packed, scale, n, k, bias=None, order=None, rows=None):
    return oracle.linear_int4_rows(x, packed, scale, n, k, order=order, rows=rows)


def _mutant(**over):
    impl = oracle_impl()
    for key, val in over.items():
        setattr(impl, key, val)
    return impl


MUTANTS = {
    "scale_amax_over_8": lambda: _mutant(quantize=lambda w: _quantize_variant(w, qmax=8)),
    "zero_row_scale_one": lambda: _mutant(quantize=lambda w: _quantize_variant(w, zero_scale=1.0)),
    "rint_half_away": lambda: _mutant(quantize=lambda w: _quantize_variant(
        w, rnd=lambda a: np.trunc(a + np.copysign(np.float32(0.5), a)))),
    "pack_nibbles_swapped": lambda: _mutant(pack=_pack_swapped),
    "linear_bias_dropped": lambda: _mutant(linear=_linear_no_bias),
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
