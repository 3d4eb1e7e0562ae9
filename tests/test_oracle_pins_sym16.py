"""Pins for the oracle's signed int4 format with float16 scales (R10).

tinyllm L8.5, "Quantization: int8, int4 group (packed), fp8, KV quant":
section 2 "Principles" (int4 per group: s16 = float16(amax / 7), codes
rint(W / s16) against the stored float16 value, zero and underflowing groups
give codes 0, a float16 overflow is refused; packing as 4-bit two's
complement, even column in the low nibble), section 3 "Worked example by
hand", and the planted mistakes of its test list (quantizing against the
float32 scale, writing an overflowing float16 scale).

As in test_oracle_pins.py, every check takes an implementation namespace, so
the same checks run against the oracle (which must pass) and against planted
mistakes (each must fail at least one check).
"""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from conftest import load_golden, parse_nums


# ---------------------------------------------------------------------------
# Exact helpers, independent of the oracle
# ---------------------------------------------------------------------------

def _nearest(fr: Fraction, dtype) -> float:
    """Correctly rounded value of a rational in a binary float type (ties to even)."""
    c = np.array(float(fr), dtype=dtype)
    cands = {c.item(), np.nextafter(c, dtype(np.inf)).item(), np.nextafter(c, dtype(-np.inf)).item()}
    best = None
    for cand in sorted(cands):
        if not np.isfinite(cand):
            continue
        bits = int(np.array(cand, dtype=dtype).view(np.uint16 if dtype == np.float16 else np.uint32))
        key = (abs(Fraction(cand) - fr), bits & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def _round_even(fr: Fraction) -> int:
    return round(fr)   # Fraction rounds halves to even


def _expect_group(wrow):
    """Codes and float16 scale of one group by the page's rule, in exact arithmetic."""
    amax = max(abs(Fraction(float(v))) for v in wrow)
    q32 = _nearest(amax / 7, np.float32)
    if q32 >= 65520:          # float16 overflow: values from 65520 up round to infinity
        return None, None
    s16 = _nearest(Fraction(q32), np.float16)
    if s16 == 0:
        return [0] * len(wrow), 0.0
    codes = []
    for v in wrow:
        quot = _nearest(Fraction(float(v)) / Fraction(s16), np.float32)
        codes.append(max(-8, min(7, _round_even(Fraction(quot)))))
    return codes, s16


def oracle_impl():
    return SimpleNamespace(
        quantize=oracle.quantize_int4_sym_f16,
        pack=oracle.pack_int4,
        unpack=oracle.unpack_int4,
        dequantize=oracle.dequantize_int4_sym_f16,
        linear=oracle.linear_int4_sym_f16,
    )


# ---------------------------------------------------------------------------
# Checks
# ---------------------------------------------------------------------------

def check_worked_example(impl):
    g = load_golden("symmetric_int4_group4_rows.txt")
    w = np.array([[float(v) for v in parse_nums(g["row0_w"])],
                  [float(v) for v in parse_nums(g["row1_w"])]], dtype=np.float32)
    c, s = impl.quantize(w, 4)
    want_c = [[int(v) for v in parse_nums(g["row0_codes"])], [int(v) for v in parse_nums(g["row1_codes"])]]
    assert np.array_equal(np.asarray(c), want_c)
    assert np.asarray(s).dtype == np.float16
    assert np.array_equal(np.asarray(s, np.float32).ravel(), [float(v) for v in parse_nums(g["scale"])])
    packed = impl.pack(c)
    want_b = [[int(v, 16) for v in g["row0_bytes_hex"].split()],
              [int(v, 16) for v in g["row1_bytes_hex"].split()]]
    assert np.array_equal(np.asarray(packed), want_b)
    w_hat = impl.dequantize(packed, s, 2, 4, 4)
    want_w = [[float(v) for v in parse_nums(g["row0_w_hat"])], [float(v) for v in parse_nums(g["row1_w_hat"])]]
    assert np.array_equal(w_hat, np.asarray(want_w, np.float32))
    assert np.max(np.abs(w_hat.astype(np.float64) - w.astype(np.float64))) == float(g["max_abs_error"])


def check_tie_against_stored_scale(impl):
    # amax / 7 = 1.0003 in float32, stored as float16 1.0: 3.5 stored scales is
    # an exact tie (to 4); against the float32 quotient it would be 3.4989 (3).
    w = np.array([[7.0021, 3.5, -3.5, 2.5, 0.5, -0.5, 1.5, 0.0]], dtype=np.float32)
    c, s = impl.quantize(w, 8)
    assert np.asarray(s, np.float32).ravel().tolist() == [1.0]
    assert np.asarray(c).ravel().tolist() == [7, 4, -4, 2, 0, 0, 2, 0]


def check_bruteforce(impl):
    rng = np.random.default_rng(7)
    for trial in range(60):
        group = [2, 4, 8, 16][trial % 4]
        scale = 10.0 ** rng.uniform(-3, 2)
        w = (rng.standard_normal((3, 2 * group)) * scale).astype(np.float32)
        if trial % 5 == 0:
            w[0, :group] = 0.0                       # an all-zero group
        c, s = impl.quantize(w, group)
        c, s = np.asarray(c), np.asarray(s, np.float32)
        for r in range(3):
            for gi in range(2):
                codes, s16 = _expect_group(w[r, gi * group:(gi + 1) * group])
                assert s[r, gi] == s16, (trial, r, gi)
                assert c[r, gi * group:(gi + 1) * group].tolist() == codes, (trial, r, gi)


def check_zero_tiny_overflow(impl):
    w = np.zeros((1, 4), np.float32)
    c, s = impl.quantize(w, 4)
    assert np.all(np.asarray(c) == 0) and np.asarray(s, np.float32)[0, 0] == 0.0
    tiny = np.full((1, 4), 1e-9, np.float32)              # amax / 7 below the float16 range
    c, s = impl.quantize(tiny, 4)
    assert np.all(np.asarray(c) == 0) and np.asarray(s, np.float32)[0, 0] == 0.0
    w_hat = impl.dequantize(impl.pack(c), s, 1, 4, 4)
    assert np.all(np.isfinite(w_hat)) and np.all(w_hat == 0)
    with pytest.raises(ValueError):
        impl.quantize(np.full((1, 4), 1e6, np.float32), 4)   # 1e6 / 7 overflows float16
    with pytest.raises(ValueError):
        impl.quantize(np.array([[0.0, np.nan, 1.0, 2.0]], np.float32), 4)


def check_half_step(impl):
    rng = np.random.default_rng(11)
    for group in (16, 32, 64):
        for log_s in np.linspace(-3, 2, 11):
            w = (rng.standard_normal((4, 4 * group)) * 10.0 ** log_s).astype(np.float32)
            c, s = impl.quantize(w, group)
            s32 = np.repeat(np.asarray(s, np.float32), group, axis=1).astype(np.float64)
            err = np.abs(np.asarray(c, np.float64) * s32 - w.astype(np.float64))
            assert np.all(err <= s32 / 2), (group, log_s)


def check_pack_exhaustive(impl):
    pairs = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], dtype=np.int8)
    packed = np.asarray(impl.pack(pairs)).ravel()
    assert len(set(packed.tolist())) == 256
    for (a, b), byte in zip(pairs.tolist(), packed.tolist()):
        assert byte == ((a & 0xF) | ((b & 0xF) << 4))
    assert np.array_equal(np.asarray(impl.unpack(packed[:, None])), pairs)
    every = np.arange(256, dtype=np.uint8)[:, None]
    assert np.array_equal(np.asarray(impl.pack(impl.unpack(every))), every)
    assert impl.pack(np.array([[-1, 0]], np.int8)).ravel().tolist() == [0x0F]
    assert impl.pack(np.array([[-8, 7]], np.int8)).ravel().tolist() == [0x78]
    for bad in ([[8, 0]], [[-9, 0]], [[1, 2, 3]]):
        with pytest.raises(ValueError):
            impl.pack(np.array(bad))


def check_dequant_exact(impl):
    rng = np.random.default_rng(3)
    n, k, g = 5, 64, 16
    c = rng.integers(-8, 8, size=(n, k)).astype(np.int8)
    s16 = (rng.uniform(0.01, 2.0, size=(n, k // g))).astype(np.float16)
    packed = impl.pack(c)
    w = impl.dequantize(packed, s16, n, k, g)
    want = c.astype(np.float64) * np.repeat(s16.astype(np.float64), g, axis=1)
    assert w.dtype == np.float32 and np.array_equal(w.astype(np.float64), want)
    bits = impl.dequantize(packed, s16, n, k, g, out="bf16")
    ref = want.astype(np.float32).view(np.uint32).astype(np.uint64)
    rb = ((ref + 0x7FFF + ((ref >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(np.asarray(bits), rb)


def _exact_linear(x, c, s16, group, bias, order):
    m, k = x.shape
    n = c.shape[0]
    xs = [[Fraction(float(v)) for v in row] for row in x]
    if order is not None:
        xs = [[row[int(o)] for o in order] for row in xs]
    out = np.empty((m, n))
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                acc += xs[i][t] * int(c[j, t]) * Fraction(float(s16[j, t // group]))
            if bias is not None:
                acc += Fraction(float(bias[j]))
            out[i, j] = float(acc)
    return out


def check_linear_exact(impl):
    rng = np.random.default_rng(5)
    for m, n, k, g, with_bias, with_order in ((1, 3, 8, 4, False, False), (2, 4, 16, 8, True, True),
                                              (3, 2, 12, 2, True, False)):
        c = rng.integers(-8, 8, size=(n, k)).astype(np.int8)
        s16 = rng.uniform(0.05, 1.5, size=(n, k // g)).astype(np.float16)
        x = rng.standard_normal((m, k)).astype(np.float32)
        bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
        order = rng.permutation(k).astype(np.int32) if with_order else None
        y = impl.linear(x, impl.pack(c), s16, n, k, g, bias=bias, order=order)
        want = _exact_linear(x, c, s16, g, bias, order)
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12), (m, n, k, g)
    # one-hot x gives the dequantized column
    c = rng.integers(-8, 8, size=(6, 8)).astype(np.int8)
    s16 = np.full((6, 2), 0.5, np.float16)
    for j in range(8):
        x = np.zeros((1, 8), np.float32)
        x[0, j] = 1.0
        y = impl.linear(x, impl.pack(c), s16, 6, 8, 4)
        assert np.array_equal(y[0], c[:, j] * 0.5)


def check_shape_rules(impl):
    w = np.ones((2, 12), np.float32)
    for bad_group in (5, 3):      # does not divide; odd
        with pytest.raises(ValueError):
            impl.quantize(w, bad_group)
    with pytest.raises(ValueError):
        impl.quantize(np.ones(8, np.float32), 4)


ALL_CHECKS = [check_worked_example, check_tie_against_stored_scale, check_bruteforce,
              check_zero_tiny_overflow, check_half_step, check_pack_exhaustive,
              check_dequant_exact, check_linear_exact, check_shape_rules]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle_impl())


# ---------------------------------------------------------------------------
# Planted mistakes (test-only copies, each with one deviation)
# ---------------------------------------------------------------------------

def _quantize_variant(w, group, qmax=7, f32_scale=False, zero_scale=0.0, rnd=np.rint, clamp=(-8, 7)):
    w = np.asarray(w, np.float32)
    if w.ndim != 2 or w.shape[1] % group or group % 2 or not np.all(np.isfinite(w)):
        raise ValueError("bad input")
    n, k = w.shape
    wg = w.reshape(n, k // group, group)
    q32 = np.abs(wg).max(-1) / np.float32(qmax)
    with np.errstate(over="ignore"):
        s16 = q32.astype(np.float16)
    if not np.all(np.isfinite(s16)):
        raise ValueError("overflow")
    s = q32 if f32_scale else s16.astype(np.float32)
    live = s16.astype(np.float32) > 0
    c = np.clip(rnd(wg / np.where(live, s, np.float32(1))[..., None]), *clamp)
    c = np.where(live[..., None], c, 0)
    s16 = np.where(live, s16, np.float16(zero_scale)).astype(np.float16)
    return c.astype(np.int8).reshape(n, k), s16


def _pack_offset(c):
    c = np.asarray(c)
    if c.shape[-1] % 2 or (c.size and (c.min() < -8 or c.max() > 7)):
        raise ValueError("bad")
    return oracle.pack_uint4((c.astype(np.int16) + 8).astype(np.uint8))


def _pack_swapped(c):
    c = np.asarray(c)
    if c.shape[-1] % 2:
        raise ValueError("bad")
    sw = c.copy()
    sw[..., 0::2], sw[..., 1::2] = c[..., 1::2], c[..., 0::2]
    return oracle.pack_int4(sw)


def _unpack_unsigned(p):
    return oracle.unpack_uint4(p).astype(np.int8)


def _linear_no_bias(x, packed, scale16, n, k, group, bias=None, order=None, rows=None):
    return oracle.linear_int4_sym_f16(x, packed, scale16, n, k, group, order=order, rows=rows)


def _linear_scatter(x, packed, scale16, n, k, group, bias=None, order=None, rows=None):
    if order is not None:
        inv = np.empty_like(np.asarray(order))
        inv[np.asarray(order)] = np.arange(len(order))
        order = inv
    return oracle.linear_int4_sym_f16(x, packed, scale16, n, k, group, bias=bias, order=order, rows=rows)


def _mutant(**over):
    impl = oracle_impl()
    for key, val in over.items():
        setattr(impl, key, val)
    return impl


MUTANTS = {
    "s07_quotient_against_float32_scale": lambda: _mutant(
        quantize=lambda w, g=32: _quantize_variant(w, g, f32_scale=True)),
    "scale_amax_over_8": lambda: _mutant(quantize=lambda w, g=32: _quantize_variant(w, g, qmax=8)),
    "zero_group_scale_one": lambda: _mutant(quantize=lambda w, g=32: _quantize_variant(w, g, zero_scale=1.0)),
    "rint_half_away": lambda: _mutant(quantize=lambda w, g=32: _quantize_variant(
        w, g, rnd=lambda a: np.trunc(a + np.copysign(np.float32(0.5), a)))),
    "codes_clamped_to_7": lambda: _mutant(quantize=lambda w, g=32: _quantize_variant(w, g, clamp=(-7, 6))),
    "pack_offset_binary": lambda: _mutant(pack=_pack_offset),
    "pack_nibbles_swapped": lambda: _mutant(pack=_pack_swapped),
    "unpack_without_sign_extension": lambda: _mutant(unpack=_unpack_unsigned),
    "linear_bias_dropped": lambda: _mutant(linear=_linear_no_bias),
    "linear_order_scatter": lambda: _mutant(linear=_linear_scatter),
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
