"""Pins for the oracle's MXFP4 functions (R11).

linnet docs "Quantization" (std.quant table, dequantize_mxfp4: E2M1 values in
blocks of 32, one E8M0 scale byte a block; the packing sentence: even element
in the low nibble) and tinyllm L8.5 section 2 "MXFP4" (a power-of-two scale X
per block of 32; elements 0, 0.5, 1, 1.5, 2, 3, 4, 6 times X; values above 6X
saturate, every element within 2X; 4.25 bits a weight) and its mutant list
(block size ignored, a byte counted per code).  The choice of X follows the
OCP Microscaling rule the page cites: X = 2^(floor(log2 amax) - 2).

Each check takes an implementation namespace; the oracle must pass every
check and each planted mistake must fail at least one.
"""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest

import oracle

MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _expect_code(v: Fraction, negative: bool) -> int:
    """Nearest E2M1 magnitude of |v| (exact), ties to the even code, saturating at 6."""
    a = min(abs(v), Fraction(6))
    dists = [abs(a - m) for m in MAGS]
    best = min(dists)
    cands = [i for i, d in enumerate(dists) if d == best]
    idx = next((i for i in cands if i % 2 == 0), cands[0])
    return idx + (8 if negative else 0)


def _expect_block(ws):
    amax = max(abs(Fraction(float(v))) for v in ws)
    if amax == 0:
        return [8 if np.signbit(v) else 0 for v in ws], 0
    j = 0                                         # floor(log2 amax), exactly
    while Fraction(2) ** (j + 1) <= amax:
        j += 1
    while Fraction(2) ** j > amax:
        j -= 1
    e = max(0, min(254, j - 2 + 127))
    x = Fraction(2) ** (e - 127)
    return [_expect_code(Fraction(float(v)) / x, bool(np.signbit(v))) for v in ws], e


def _value(code: int, e: int) -> Fraction:
    v = MAGS[code & 7] * Fraction(2) ** (e - 127)
    return -v if code & 8 else v


def oracle_impl():
    return SimpleNamespace(quantize=oracle.quantize_mxfp4, pack=oracle.pack_uint4,
                           unpack=oracle.unpack_uint4, dequantize=oracle.dequantize_mxfp4,
                           linear=oracle.linear_mxfp4)


# ---------------------------------------------------------------------------
# Checks
# ---------------------------------------------------------------------------

def check_hand_block(impl):
    # amax 7 -> floor(log2 7) = 2 -> X = 1 (E8M0 127).  Ties: 0.25 -> 0, 0.75 -> 1,
    # 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4 (even codes); 7 and 6.5 saturate
    # to 6; -0.1 rounds to -0 (code 8), -0.3 to -0.5 (code 9).
    w = np.zeros((1, 32), np.float32)
    w[0, :12] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.1, -0.3, 6.5, 0.0]
    c, e = impl.quantize(w)
    assert np.asarray(e).ravel().tolist() == [127]
    assert np.asarray(c)[0, :12].tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 8, 9, 7, 0]
    blocks = impl.pack(c)
    assert np.asarray(blocks)[0, :6].tolist() == [0x20, 0x42, 0x64, 0x76, 0x98, 0x07]
    w_hat = impl.dequantize(blocks, e, 1, 32)
    assert w_hat[0, :12].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -0.0, -0.5, 6.0, 0.0]


def check_scale_choice(impl):
    # amax exactly 4 -> X = 1; just below 4 -> X = 1/2; 1e-40 (float32 subnormal) -> E8M0 0
    for amax, e_want in ((4.0, 127), (np.nextafter(np.float32(4), np.float32(0)), 126), (1.0, 125),
                         (1e-40, 0), (3.0e38, 252)):
        w = np.zeros((1, 32), np.float32)
        w[0, 5] = amax
        _, e = impl.quantize(w)
        assert int(np.asarray(e).ravel()[0]) == e_want, (amax, e)


def check_zero_block(impl):
    w = np.zeros((2, 64), np.float32)
    w[1, 32:] = 1.0
    c, e = impl.quantize(w)
    assert np.asarray(e).ravel().tolist()[:3] == [0, 0, 0]
    assert np.all(np.asarray(c)[0] == 0)
    with pytest.raises(ValueError):
        impl.quantize(np.array([[np.inf] + [0.0] * 31], np.float32))


def check_bruteforce(impl):
    rng = np.random.default_rng(13)
    for trial in range(40):
        scale = 10.0 ** rng.uniform(-6, 4)
        w = (rng.standard_normal((2, 64)) * scale).astype(np.float32)
        if trial % 4 == 0:
            w[0, 3] = np.float32(-0.0)
        c, e = impl.quantize(w)
        c, e = np.asarray(c), np.asarray(e)
        for r in range(2):
            for b in range(2):
                codes, eb = _expect_block(w[r, 32 * b:32 * (b + 1)])
                assert int(e[r, b]) == eb, (trial, r, b)
                assert c[r, 32 * b:32 * (b + 1)].tolist() == codes, (trial, r, b)


def check_error_within_2x(impl):
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    c, e = impl.quantize(w)
    w_hat = impl.dequantize(impl.pack(c), e, 16, 256).astype(np.float64)
    x = np.repeat(np.ldexp(1.0, np.asarray(e, np.int64) - 127), 32, axis=1)
    err = np.abs(w_hat - w.astype(np.float64))
    assert np.all(err <= 2 * x)
    small = np.abs(w) <= 4 * x                    # below the 4X..6X gap the step is at most X
    assert np.all(err[small] <= x[small] / 2 + 0)


def check_layout_and_size(impl):
    w = np.ones((3, 96), np.float32)
    c, e = impl.quantize(w)
    blocks = impl.pack(c)
    assert np.asarray(e).shape == (3, 3)
    assert np.asarray(blocks).shape == (3, 48)
    bits = (np.asarray(blocks).nbytes + np.asarray(e).nbytes) * 8
    assert bits == 4.25 * 3 * 96                  # 4 + 8/32 bits a weight


def check_dequant_exact(impl):
    rng = np.random.default_rng(19)
    n, k = 6, 128
    c = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    e = rng.integers(100, 150, size=(n, k // 32)).astype(np.uint8)
    blocks = impl.pack(c)
    got = impl.dequantize(blocks, e, n, k)
    for r in range(n):
        for j in range(k):
            assert Fraction(float(got[r, j])) == _value(int(c[r, j]), int(e[r, j // 32])), (r, j)
    bits = impl.dequantize(blocks, e, n, k, out="bf16")
    ref = got.view(np.uint32).astype(np.uint64)
    assert np.array_equal(np.asarray(bits), ((ref + 0x7FFF + ((ref >> 16) & 1)) >> 16).astype(np.uint16))


def check_linear_exact(impl):
    rng = np.random.default_rng(23)
    for m, n, k, with_bias in ((1, 3, 32, False), (2, 4, 64, True), (3, 2, 96, True)):
        c = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
        e = rng.integers(120, 130, size=(n, k // 32)).astype(np.uint8)
        x = rng.standard_normal((m, k)).astype(np.float32)
        bias = rng.standard_normal(n).astype(np.float32) if with_bias else None
        y = impl.linear(x, impl.pack(c), e, n, k, bias=bias)
        for i in range(m):
            for j in range(n):
                acc = sum(Fraction(float(x[i, t])) * _value(int(c[j, t]), int(e[j, t // 32])) for t in range(k))
                if bias is not None:
                    acc += Fraction(float(bias[j]))
                assert abs(y[i, j] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc))), (m, i, j)
    # one-hot input picks a column
    c = rng.integers(0, 16, size=(5, 32)).astype(np.uint8)
    e = np.full((5, 1), 127, np.uint8)
    for j in (0, 7, 31):
        x = np.zeros((1, 32), np.float32)
        x[0, j] = 1.0
        y = impl.linear(x, impl.pack(c), e, 5, 32)
        assert [Fraction(float(v)) for v in y[0]] == [_value(int(c[r, j]), 127) for r in range(5)]


ALL_CHECKS = [check_hand_block, check_scale_choice, check_zero_block, check_bruteforce,
              check_error_within_2x, check_layout_and_size, check_dequant_exact, check_linear_exact]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle_impl())


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _quantize_variant(w, block=32, emax=2, bias=127, ties_away=False, keep_neg_zero=True,
                      saturate=True):
    w = np.asarray(w, np.float32)
    if w.ndim != 2 or w.shape[1] % block or not np.all(np.isfinite(w)):
        raise ValueError("bad input")
    n, k = w.shape
    wb = w.reshape(n, k // block, block).astype(np.float64)
    amax = np.abs(wb).max(-1)
    _, ex = np.frexp(amax)
    e = np.where(amax > 0, np.clip(ex - 1 - emax + bias, 0, 254), 0).astype(np.int64)
    x = np.ldexp(1.0, e - bias)
    v = wb / x[..., None]
    mags = np.array(oracle.E2M1_VALUES)
    a = np.abs(v)
    if saturate:
        a = np.minimum(a, 6.0)
    d = np.abs(a[..., None] - mags)
    best = d.min(-1, keepdims=True)
    cand = d == best
    if ties_away:
        idx = 7 - np.argmax(cand[..., ::-1], axis=-1)
    else:
        even = cand & (np.arange(8) % 2 == 0)
        idx = np.where(even.any(-1), np.argmax(even, -1), np.argmax(cand, -1))
    neg = np.signbit(v) if keep_neg_zero else (v < 0) & (idx > 0)
    codes = (idx + np.where(neg, 8, 0)).astype(np.uint8).reshape(n, k)
    if block != 32:   # scales per block of the wrong size, laid out as [N, K/block]
        return codes, e.astype(np.uint8)
    return codes, e.astype(np.uint8)


def _pack_swapped(q):
    q = np.asarray(q)
    sw = q.copy()
    sw[..., 0::2], sw[..., 1::2] = q[..., 1::2], q[..., 0::2]
    return oracle.pack_uint4(sw)


def _linear_no_bias(x, blocks, scales, n, k, bias=None, rows=None):
    return oracle.linear_mxfp4(x, blocks, scales, n, k, rows=rows)


def _mutant(**over):
    impl = oracle_impl()
    for key, val in over.items():
        setattr(impl, key, val)
    return impl


MUTANTS = {
    "s13_block_of_16": lambda: _mutant(quantize=lambda w: _quantize_variant(w, block=16)),
    "scale_exponent_minus_3": lambda: _mutant(quantize=lambda w: _quantize_variant(w, emax=3)),
    "scale_exponent_minus_1": lambda: _mutant(quantize=lambda w: _quantize_variant(w, emax=1)),
    "e8m0_bias_128": lambda: _mutant(quantize=lambda w: _quantize_variant(w, bias=128)),
    "ties_to_larger_code": lambda: _mutant(quantize=lambda w: _quantize_variant(w, ties_away=True)),
    "negative_zero_dropped": lambda: _mutant(quantize=lambda w: _quantize_variant(w, keep_neg_zero=False)),
    "nibbles_swapped": lambda: _mutant(pack=_pack_swapped),
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
