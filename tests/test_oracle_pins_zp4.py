"""Pins for the oracle's packed 4-bit zero points (R15).

linnet "Quantization": Int4GroupLinear's layout is ONNX Runtime's MatMulNBits,
whose zero points are 4-bit values two a byte.  The pins: a hand row of three
groups ([1, 2, 3] -> 0x21 0x03, the padding nibble 0); every pair of values
round-trips; an odd group count pads only the row's last byte; refusals; and
the layer over packed zero points against exact rational arithmetic.
"""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest

import oracle


def oracle_impl():
    return SimpleNamespace(pack=oracle.pack_zero_points, unpack=oracle.unpack_zero_points,
                           linear=oracle.linear_int4_groups_zp4)


def check_hand_rows(impl):
    assert np.asarray(impl.pack(np.array([[1, 2, 3]]))).tolist() == [[0x21, 0x03]]
    assert np.asarray(impl.pack(np.array([[15, 0], [0, 15]]))).tolist() == [[0x0F], [0xF0]]
    assert np.asarray(impl.unpack(np.array([[0x21, 0xF3]], np.uint8), 1, 3)).tolist() == [[1, 2, 3]]


def check_all_pairs_round_trip(impl):
    a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    z = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.uint8)        # 256 rows of two groups
    p = np.asarray(impl.pack(z))
    assert p.shape == (256, 1) and sorted(p[:, 0].tolist()) == list(range(256))
    assert np.all(p[:, 0] == z[:, 0] + 16 * z[:, 1])
    assert np.array_equal(impl.unpack(p, 256, 2), z)


def check_odd_group_count(impl):
    rng = np.random.default_rng(3)
    for ng in (1, 3, 7, 33):
        z = rng.integers(0, 16, size=(5, ng)).astype(np.uint8)
        p = np.asarray(impl.pack(z))
        assert p.shape == (5, (ng + 1) // 2)
        assert np.all(p[:, -1] >> 4 == 0) if ng % 2 else True
        assert np.array_equal(impl.unpack(p, 5, ng), z)


def check_refusals(impl):
    for bad in (np.array([[16, 0]]), np.array([[-1, 0]]), np.array([1, 2])):
        with pytest.raises(ValueError):
            impl.pack(bad)


def check_linear_exact(impl):
    rng = np.random.default_rng(7)
    m, n, k, g = 2, 3, 24, 8
    q = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    sc = rng.uniform(0.01, 1.0, size=(n, k // g)).astype(np.float32)
    z = rng.integers(0, 16, size=(n, k // g)).astype(np.uint8)
    x = rng.standard_normal((m, k)).astype(np.float32)
    bias = rng.standard_normal(n).astype(np.float32)
    zp = oracle.pack_zero_points(z)                   # the reference packing, pinned above
    y = impl.linear(x, oracle.pack_uint4(q), sc, zp, n, k, g, bias=bias)
    for i in range(m):
        for j in range(n):
            acc = Fraction(float(bias[j]))
            for c in range(k):
                acc += Fraction(float(x[i, c])) * (int(q[j, c]) - int(z[j, c // g])) * Fraction(float(sc[j, c // g]))
            assert abs(y[i, j] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))


ALL_CHECKS = [check_hand_rows, check_all_pairs_round_trip, check_odd_group_count, check_refusals, check_linear_exact]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle_impl())


def _pack_swapped(z):
    z = np.asarray(z)
    p = oracle.pack_zero_points(z)
    return ((p >> 4) | (p << 4)).astype(np.uint8)


def _pack_pad8(z):
    z = np.asarray(z)
    if z.ndim == 2 and z.shape[1] % 2:
        z = np.concatenate([z, np.full((z.shape[0], 1), 8)], axis=1)
    return oracle.pack_zero_points(z)


def _unpack_high_first(p, n, ng):
    p = np.asarray(p, np.uint8).reshape(n, (ng + 1) // 2)
    out = np.empty((n, 2 * p.shape[1]), np.uint8)
    out[:, 0::2], out[:, 1::2] = p >> 4, p & 15
    return out[:, :ng]


def _linear_zero_ignored(x, packed, scale, zp, n, k, group, bias=None, order=None, rows=None):
    return oracle.linear_int4_groups(x, packed, scale, np.zeros((n, k // group), np.uint8), n, k, group,
                                     bias=bias, order=order, rows=rows)


def _mutant(**over):
    impl = oracle_impl()
    for key, val in over.items():
        setattr(impl, key, val)
    return impl


MUTANTS = {
    "nibbles_swapped": lambda: _mutant(pack=_pack_swapped),
    "padding_nibble_8": lambda: _mutant(pack=_pack_pad8),
    "unpack_high_nibble_first": lambda: _mutant(unpack=_unpack_high_first),
    "linear_ignores_zero_points": lambda: _mutant(linear=_linear_zero_ignored),
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
