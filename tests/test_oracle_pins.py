"""Pins for the CPU oracle: worked examples, exact arithmetic, invariants, mutants.

Every check here takes an implementation namespace so the same check can be
run against the oracle (it must pass) and against deliberately broken copies
of it (each must be caught by at least one check).  The broken copies follow
the planted-bug list of tinyllm L8.5 section 5 ("Pitfalls") where it applies
to the unsigned group layout.
"""
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden, parse_nums


# ---------------------------------------------------------------------------
# Exact-arithmetic helpers (independent of the oracle)
# ---------------------------------------------------------------------------

def frac(v):
    return Fraction(float(v))


def nearest_f32(fr: Fraction) -> np.float32:
    """Correctly rounded float32 of a rational (ties to even), found by exact comparison."""
    c = np.float32(float(fr))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = None
    for cand in sorted(cands):
        dist = abs(Fraction(float(cand)) - fr)
        key = (dist, int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def round_even(fr: Fraction) -> int:
    return round(fr)   # Fraction.__round__ without ndigits rounds halves to even


def oracle_impl():
    return SimpleNamespace(
        rint_half_even=oracle.rint_half_even,
        quantize_groups=oracle.quantize_groups,
        pack_uint4=oracle.pack_uint4,
        unpack_uint4=oracle.unpack_uint4,
        dequantize_int4_groups=oracle.dequantize_int4_groups,
        linear_int4_groups=oracle.linear_int4_groups,
        bf16_round_bits=oracle.bf16_round_bits,
        prepare_int4=oracle.prepare_int4,
        unprepare_int4=oracle.unprepare_int4,
    )


# ---------------------------------------------------------------------------
# Checks
# ---------------------------------------------------------------------------

def check_rint_ties(impl):
    g = load_golden("int8_ties_scale1.txt")
    vals = np.array([float(v) for v in parse_nums(g["values"])])
    want = np.array([float(v) for v in parse_nums(g["rounded"])])
    got = impl.rint_half_even(vals)
    assert np.array_equal(got, want), (got, want)


def check_worked_example_group5(impl):
    g = load_golden("symmetric_int4_group5.txt")
    w = np.array([[float(v) for v in parse_nums(g["w"])]], dtype=np.float32)
    q, s, z = impl.quantize_groups(w, int(g["group"]), symmetric=True)
    codes = q.astype(np.int64) - z.astype(np.int64)
    want = [int(v) for v in parse_nums(g["codes"])]
    assert codes[0].tolist() == want, codes
    assert s[0, 0] == nearest_f32(Fraction(g["scale_real"]))
    w_hat = [float(c * Fraction(float(s[0, 0]))) for c in want]
    for a, b in zip(w_hat, parse_nums(g["w_hat_3dp"])):
        assert abs(a - float(b)) <= 5e-4


def check_worked_example_group4_rows(impl):
    g = load_golden("symmetric_int4_group4_rows.txt")
    w = np.array([[float(v) for v in parse_nums(g["row0_w"])],
                  [float(v) for v in parse_nums(g["row1_w"])]], dtype=np.float32)
    q, s, z = impl.quantize_groups(w, int(g["group"]), symmetric=True)
    codes = q.astype(np.int64) - z.astype(np.int64)
    assert codes[0].tolist() == [int(v) for v in parse_nums(g["row0_codes"])]
    assert codes[1].tolist() == [int(v) for v in parse_nums(g["row1_codes"])]
    assert s.ravel().tolist() == [float(v) for v in parse_nums(g["scale"])]
    # Two's-complement nibbles packed even-column-low must give the printed bytes.
    for r in (0, 1):
        nib = np.array([int(t, 16) for t in g[f"row{r}_nibbles_hex"].split()], dtype=np.uint8)
        assert np.array_equal(nib, (codes[r] & 0xF).astype(np.uint8))
        want_bytes = [int(t, 16) for t in g[f"row{r}_bytes_hex"].split()]
        assert impl.pack_uint4(nib).tolist() == want_bytes
        assert impl.unpack_uint4(np.array(want_bytes, dtype=np.uint8)).tolist() == nib.tolist()
    # Dequantize the unsigned layout and compare with the printed reconstruction.
    wh = impl.dequantize_int4_groups(impl.pack_uint4(q), s, z, 2, 4, 4, "f32")
    assert wh[0].tolist() == [float(v) for v in parse_nums(g["row0_w_hat"])]
    assert wh[1].tolist() == [float(v) for v in parse_nums(g["row1_w_hat"])]
    assert float(np.max(np.abs(wh.astype(np.float64) - w.astype(np.float64)))) == \
        float(Fraction(g["max_abs_error"]))


def check_pack_exhaustive(impl):
    lo, hi = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    pairs = np.stack([lo.ravel(), hi.ravel()], axis=-1).astype(np.uint8)   # [256, 2]
    packed = impl.pack_uint4(pairs)
    assert packed.shape == (256, 1)
    assert len(set(packed.ravel().tolist())) == 256
    assert np.array_equal(impl.unpack_uint4(packed), pairs)
    allb = np.arange(256, dtype=np.uint8).reshape(256, 1)
    assert np.array_equal(impl.pack_uint4(impl.unpack_uint4(allb)), allb)
    # the even element sits in the low nibble
    assert impl.pack_uint4(np.array([1, 0], dtype=np.uint8)).tolist() == [0x01]
    assert impl.pack_uint4(np.array([0, 1], dtype=np.uint8)).tolist() == [0x10]
    for bad in (np.array([16, 0], dtype=np.uint8), np.array([1, 2, 3], dtype=np.uint8)):
        with pytest.raises(ValueError):
            impl.pack_uint4(bad)


def _asym_expect(wrow, group):
    """Brute-force expectation for one row: exact zero, scale and nearest level."""
    out = []
    for g0 in range(0, len(wrow), group):
        grp = [frac(v) for v in wrow[g0:g0 + group]]
        mn, mx = min(grp), max(grp)
        d = mx - mn
        out.append((grp, mn, mx, d))
    return out


def check_asym_bruteforce(impl):
    rng = np.random.default_rng(7)
    cases = []
    for group in (2, 4, 8, 32, 128):
        for scale in (1e-3, 0.02, 1.0, 37.0):
            cases.append((rng.standard_normal((3, 2 * group)).astype(np.float32) * np.float32(scale), group))
    # Exact ties everywhere: range 15, zero 1 (odd), weights on the half-step grid.
    tie = np.array([[-1.0] + [v / 2 for v in range(-2, 29)] + [14.0]], dtype=np.float32)
    cases.append((tie, tie.shape[1]))
    for w, group in cases:
        q, s, z = impl.quantize_groups(w, group)
        for r in range(w.shape[0]):
            for gi, (grp, mn, mx, d) in enumerate(_asym_expect(w[r], group)):
                assert d > 0
                zexp = min(max(round_even(-15 * mn / d), 0), 15)
                assert int(z[r, gi]) == zexp, (r, gi, int(z[r, gi]), zexp)
                assert s[r, gi] == nearest_f32(d / 15)
                for e, wv in enumerate(grp):
                    dist = [abs(wv - (j - zexp) * d / 15) for j in range(16)]
                    best = min(dist)
                    cands = [j for j in range(16) if dist[j] == best]
                    got = int(q[r, gi * group + e])
                    assert got in cands, (wv, got, cands)
                    if len(cands) == 2:
                        assert (got - zexp) % 2 == 0, (wv, got, cands)


def check_symmetric_bruteforce(impl):
    rng = np.random.default_rng(11)
    for group in (2, 4, 16, 64):
        w = rng.standard_normal((4, 3 * group)).astype(np.float32) * np.float32(0.3)
        w[0, :group] = np.float32(0.5) * np.round(w[0, :group] * 8)   # ties
        q, s, z = impl.quantize_groups(w, group, symmetric=True)
        assert np.all(z == 8)
        for r in range(w.shape[0]):
            for gi in range(w.shape[1] // group):
                grp = [frac(v) for v in w[r, gi * group:(gi + 1) * group]]
                a = max(abs(v) for v in grp)
                assert s[r, gi] == nearest_f32(a / 7)
                for e, wv in enumerate(grp):
                    c = int(q[r, gi * group + e]) - 8
                    assert c == max(-7, min(7, round_even(7 * wv / a)))


def check_zero_groups(impl):
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    q, s, z = impl.quantize_groups(w, 32)
    assert s[0].tolist() == [1.0, 1.0] and s[1, 0] == 1.0
    assert z[0].tolist() == [0, 0] and int(z[1, 0]) == 0
    assert np.all(q[0] == 0) and np.all(q[1, :32] == 0)
    qs, ss, zs = impl.quantize_groups(w, 32, symmetric=True)
    assert ss[0].tolist() == [1.0, 1.0] and np.all(qs[0] == 8)


HALF_STEP_SLACK = 1 + 2.0 ** -17   # float32 rounding of the stored scale and of q*s


def _half_step_ok(impl, w, group):
    q, s, z = impl.quantize_groups(w, group)
    n, k = w.shape
    wh = impl.dequantize_int4_groups(impl.pack_uint4(q), s, z, n, k, group, "f32")
    err = np.abs(wh.astype(np.float64) - w.astype(np.float64)).reshape(n, k // group, group)
    wg = w.reshape(n, k // group, group)
    spans0 = (wg.min(-1) <= 0) & (wg.max(-1) >= 0)
    bound = s.astype(np.float64) / 2 * HALF_STEP_SLACK
    return bool(np.all(err.max(-1)[spans0] <= bound[spans0])), q, wg


def check_half_step_sweep(impl):
    rng = np.random.default_rng(3)
    for group in (32, 64, 128, 256):
        for scale in np.logspace(-3, 2, 6):
            w = (rng.standard_normal((16, 2 * group)) * scale).astype(np.float32)
            ok, q, wg = _half_step_ok(impl, w, group)
            assert ok, (group, scale)
            # the group minimum maps to code 0 whenever the group spans zero
            qg = q.reshape(wg.shape)
            mins = np.argmin(wg, axis=-1)
            assert np.all(np.take_along_axis(qg, mins[..., None], -1) == 0)


def check_noise_variance(impl):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((1024, 1024)) * 0.02).astype(np.float32)
    q, s, z = impl.quantize_groups(w, 128)
    wh = impl.dequantize_int4_groups(impl.pack_uint4(q), s, z, 1024, 1024, 128, "f32")
    r = (wh.astype(np.float64) - w).reshape(1024, 8, 128) / s.astype(np.float64)[..., None]
    assert abs(np.mean(r * r) * 12 - 1) < 0.03


def check_dequant_closed_form(impl):
    rng = np.random.default_rng(9)
    n, k, group = 8, 256, 32
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = (rng.standard_normal((n, k // group)) * 0.01).astype(np.float32)
    s[0, 0] = np.float32(3.3e-39)     # subnormal scale
    z = rng.integers(0, 16, (n, k // group), dtype=np.uint8)
    packed = impl.pack_uint4(q)
    got32 = impl.dequantize_int4_groups(packed, s, z, n, k, group, "f32")
    tq = torch.from_numpy(q.astype(np.float32)).view(n, k // group, group)
    tz = torch.from_numpy(z.astype(np.float32))[..., None]
    ts = torch.from_numpy(s)[..., None]
    want32 = ((tq - tz) * ts).reshape(n, k).numpy()   # IEEE float32 arithmetic
    assert np.array_equal(got32.view(np.uint32), want32.view(np.uint32))
    got16 = impl.dequantize_int4_groups(packed, s, z, n, k, group, "bf16")
    want16 = torch.from_numpy(want32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got16, want16)


def check_bf16_rounding(impl):
    rng = np.random.default_rng(13)
    v = rng.standard_normal(100000).astype(np.float32) * np.float32(100)
    bits = v.view(np.uint32)
    # force exact ties with both parities of the kept bit
    bits[:1000] = (bits[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    v = bits.view(np.float32)
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(impl.bf16_round_bits(v), want)


def _exact_linear(x_bits, q, s, z, group, bias, order):
    xv = [[Fraction(float(t)) for t in row] for row in oracle.bf16_bits_to_f64(x_bits)]
    m, k = len(xv), len(xv[0])
    n = q.shape[0]
    y = [[Fraction(0)] * n for _ in range(m)]
    for mi in range(m):
        xr = xv[mi] if order is None else [xv[mi][int(order[kk])] for kk in range(k)]
        for ni in range(n):
            acc = Fraction(0)
            for kk in range(k):
                g = kk // group
                acc += xr[kk] * (int(q[ni, kk]) - int(z[ni, g])) * Fraction(float(s[ni, g]))
            if bias is not None:
                acc += Fraction(float(bias[ni]))
            y[mi][ni] = acc
    return y


def check_linear_exact(impl):
    import workloads
    for (m, n, k, group, with_bias, with_order) in ((3, 6, 8, 4, True, True), (2, 8, 8, 2, True, False),
                                                    (1, 5, 12, 6, False, True), (2, 8, 8, 4, False, False)):
        w = workloads.weight(n, k, seed=17 + n, std=0.5)
        x = workloads.activations_bf16(m, k, seed=19 + k)
        b = workloads.bias(n, seed=23) if with_bias else None
        o = np.array([(5 * i + 1) % k for i in range(k)], dtype=np.int32) if with_order else None
        if o is not None:
            assert len(set(o.tolist())) == k
        q, s, z = impl.quantize_groups(w, group)
        packed = impl.pack_uint4(q)
        y = impl.linear_int4_groups(x, packed, s, z, n, k, group, bias=b, order=o)
        ye = _exact_linear(x, q, s, z, group, b, o)
        for mi in range(m):
            for ni in range(n):
                assert abs(Fraction(float(y[mi, ni])) - ye[mi][ni]) <= Fraction(1, 2 ** 40), (mi, ni)


def check_linear_onehot_and_zero(impl):
    n, k, group = 12, 64, 32
    import workloads
    w = workloads.weight(n, k, seed=29)
    q, s, z = impl.quantize_groups(w, group)
    packed = impl.pack_uint4(q)
    one = np.float32(1.0).view(np.uint32) >> np.uint32(16)
    x = np.zeros((k, k), dtype=np.uint16)
    x[np.arange(k), np.arange(k)] = one                     # rows are e_j
    y = impl.linear_int4_groups(x, packed, s, z, n, k, group)
    for j in (0, 5, 31, 32, 63):
        for ni in range(n):
            want = (int(q[ni, j]) - int(z[ni, j // group])) * Fraction(float(s[ni, j // group]))
            assert Fraction(float(y[j, ni])) == want
    # zero weights: y is exactly the bias
    b = workloads.bias(n, seed=31)
    q0, s0, z0 = impl.quantize_groups(np.zeros((n, k), np.float32), group)
    y0 = impl.linear_int4_groups(x[:3], impl.pack_uint4(q0), s0, z0, n, k, group, bias=b)
    assert np.array_equal(y0, np.broadcast_to(b.astype(np.float64), y0.shape))


def check_linear_order_and_rows(impl):
    import workloads
    m, n, k, group = 4, 40, 128, 32
    w = workloads.weight(n, k, seed=37)
    x = workloads.activations_bf16(m, k, seed=41)
    q, s, z = impl.quantize_groups(w, group)
    packed = impl.pack_uint4(q)
    ident = np.arange(k, dtype=np.int32)
    y_plain = impl.linear_int4_groups(x, packed, s, z, n, k, group)
    assert np.array_equal(impl.linear_int4_groups(x, packed, s, z, n, k, group, order=ident), y_plain)
    perm = workloads.order(k, seed=43)
    y_perm = impl.linear_int4_groups(x, packed, s, z, n, k, group, order=perm)
    assert np.array_equal(y_perm, impl.linear_int4_groups(x[:, perm], packed, s, z, n, k, group))
    rows = np.array([0, 7, 39, 12])
    assert np.array_equal(impl.linear_int4_groups(x, packed, s, z, n, k, group, rows=rows),
                          y_plain[:, rows])


def check_shape_rules(impl):
    w = np.ones((2, 12), dtype=np.float32)
    with pytest.raises(ValueError):
        impl.quantize_groups(w, 5)                          # does not divide In
    with pytest.raises(ValueError):
        impl.quantize_groups(np.ones(12, np.float32), 4)    # 1-D input
    bad = w.copy()
    bad[0, 3] = np.nan
    with pytest.raises(ValueError):
        impl.quantize_groups(bad, 4)
    q, s, z = oracle.quantize_groups(np.ones((2, 6), np.float32), 3)
    with pytest.raises(ValueError):
        impl.dequantize_int4_groups(np.zeros((2, 3), np.uint8), s, z, 2, 6, 3, "f32")   # odd group
    x = np.zeros((1, 6), dtype=np.uint16)
    with pytest.raises(ValueError):
        impl.linear_int4_groups(x, np.zeros((2, 3), np.uint8), s, z, 2, 6, 3)


def _position_ids(impl, n, k):
    """Prepare an [n, k/2] byte matrix whose entries name their own position.

    Bytes hold only 8 bits, so the position p + 1 (0 marks padding) goes
    through the permutation one base-256 digit at a time and is put back
    together afterwards.
    """
    pos = np.arange(n * (k // 2), dtype=np.int64).reshape(n, k // 2) + 1
    out = None
    for d in range(3):
        digit = ((pos >> (8 * d)) & 0xFF).astype(np.uint8)
        part = np.asarray(impl.prepare_int4(digit, n, k)).astype(np.int64) << (8 * d)
        out = part if out is None else out | part
    return out


def check_prepared_fragments(impl):
    """Prepared weights (R9): every packed byte appears exactly once, padding is
    zero, each 1 KB block is one (16-row tile, 128-input step), blocks run
    through the steps of a tile before the next tile, and the 16-byte slot l of
    a block holds 32 consecutive inputs of tile row l % 16, quarter l // 16 of
    the step (the MFMA operand order the kernels load).  Sizes include ragged
    rows and steps."""
    for n, k in ((1, 32), (16, 128), (17, 96), (33, 288), (40, 1024)):
        ids = _position_ids(impl, n, k)
        nt, ns = -(-n // 16), -(-k // 128)
        assert ids.size == nt * ns * 1024 == oracle.prepared_bytes(n, k)
        real = ids[ids > 0] - 1
        assert real.size == n * (k // 2) and np.array_equal(np.sort(real), np.arange(n * (k // 2)))
        slots = ids.reshape(nt, ns, 64, 16)
        for t in range(nt):
            for s_ in range(ns):
                for l in range(64):
                    row, quarter = 16 * t + l % 16, l // 16
                    first_byte = 64 * s_ + 16 * quarter      # inputs 128 s + 32 quarter ..
                    expect = [row * (k // 2) + first_byte + b + 1
                              if row < n and first_byte + b < k // 2 else 0 for b in range(16)]
                    assert list(slots[t, s_, l]) == expect, (n, k, t, s_, l)


def check_prepared_roundtrip(impl):
    """unprepare(prepare(p)) == p on random bytes, ragged sizes included, and a
    prepared buffer decodes to the same dequantized weights."""
    rng = np.random.default_rng(11)
    for n, k in ((3, 64), (16, 4096), (31, 160), (64, 384)):
        p = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
        pr = impl.prepare_int4(p, n, k)
        back = impl.unprepare_int4(pr, n, k)
        assert np.array_equal(np.asarray(back).reshape(n, k // 2), p)
    with pytest.raises(ValueError):
        impl.prepare_int4(np.zeros((2, 24), np.uint8), 2, 48)     # k not a multiple of 32


ALL_CHECKS = [
    check_rint_ties, check_worked_example_group5, check_worked_example_group4_rows,
    check_pack_exhaustive, check_asym_bruteforce, check_symmetric_bruteforce,
    check_zero_groups, check_half_step_sweep, check_noise_variance,
    check_dequant_closed_form, check_bf16_rounding, check_linear_exact,
    check_linear_onehot_and_zero, check_linear_order_and_rows, check_shape_rules,
    check_prepared_fragments, check_prepared_roundtrip,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(oracle_impl())


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one check
# ---------------------------------------------------------------------------

def _quantize_variant(w, group, symmetric=False, rnd=np.rint, qden_scale=15, zero_inside=False,
                      f32_quotient=False):
    """The asymmetric quantizer with one planted deviation (test-only copy)."""
    if symmetric:
        if f32_quotient:
            w = np.asarray(w, np.float32)
            n, k = w.shape
            wg = w.reshape(n, k // group, group)
            a = np.abs(wg).max(-1)
            s = np.where(a > 0, a / np.float32(7), np.float32(1)).astype(np.float32)
            c = np.clip(np.rint(wg / s[..., None]), -7, 7)
            return (c + 8).astype(np.uint8).reshape(n, k), s, np.full((n, k // group), 8, np.uint8)
        return oracle.quantize_groups(w, group, symmetric=True)
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % group or not np.all(np.isfinite(w)):
        raise ValueError("bad input")
    n, k = w.shape
    wg = w.reshape(n, k // group, group).astype(np.float64)
    mn, mx = wg.min(-1), wg.max(-1)
    d = mx - mn
    flat = d == 0
    ds = np.where(flat, 1.0, d)
    scale = np.where(flat, 1.0, ds / qden_scale).astype(np.float32)
    zero = np.clip(np.where(flat, rnd(-mn), rnd(-15 * mn / ds)), 0, 15)
    if zero_inside:
        r = rnd(15 * wg / ds[..., None] + zero[..., None])
        q = np.clip(np.where(flat[..., None], rnd(wg) + zero[..., None], r), 0, 15)
    else:
        r = np.where(flat[..., None], rnd(wg), rnd(15 * wg / ds[..., None]))
        q = np.clip(r + zero[..., None], 0, 15)
    return q.astype(np.uint8).reshape(n, k), scale, zero.astype(np.uint8)


def _mutant(**over):
    impl = oracle_impl()
    for key, val in over.items():
        setattr(impl, key, val)
    return impl


def _pack_swapped(q):
    q = np.asarray(q)
    if q.shape[-1] % 2 or (q.size and q.max() > 15):
        raise ValueError("bad")
    sw = q.copy()
    sw[..., 0::2], sw[..., 1::2] = q[..., 1::2], q[..., 0::2]
    return oracle.pack_uint4(sw)


def _linear_variant(x, packed, scale, zero, n, k, group, bias=None, order=None, rows=None,
                    drop_bias=False, transpose_w=False, wrong_axis=False, scatter=False):
    if group % 2 or k % group:
        raise ValueError("bad group")
    xv = oracle.bf16_bits_to_f64(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, np.float64)
    if order is not None:
        if scatter:
            xs = np.empty_like(xv)
            xs[:, np.asarray(order)] = xv
            xv = xs
        else:
            xv = xv[:, np.asarray(order)]
    q = oracle.unpack_uint4(np.asarray(packed).reshape(n, k // 2)).astype(np.float64)
    s = np.asarray(scale, np.float64).reshape(n, k // group)
    z = np.asarray(zero, np.float64).reshape(n, k // group)
    if wrong_axis:
        srep = np.tile(s, (1, group))          # groups repeated across the row, not expanded
        zrep = np.tile(z, (1, group))
    else:
        srep = np.repeat(s, group, axis=1)
        zrep = np.repeat(z, group, axis=1)
    wh = (q - zrep) * srep
    y = xv @ (wh if transpose_w and wh.shape[0] == wh.shape[1] else wh.T)
    if bias is not None and not drop_bias:
        y = y + np.asarray(bias, np.float64)[None, :]
    if rows is not None:
        y = y[:, np.asarray(rows)]
    return y


def _dequant_odd_ok(packed, scale, zero, n, k, group, out="f32"):
    if k % group:
        raise ValueError("bad")
    q = oracle.unpack_uint4(np.asarray(packed).reshape(n, -1))[:, :k].astype(np.float64)
    w = (q - np.repeat(np.asarray(zero, np.float64), group, 1)) * np.repeat(np.asarray(scale, np.float64), group, 1)
    return w.astype(np.float32)


MUTANTS = {
    "s01_nibbles_swapped": lambda: _mutant(pack_uint4=_pack_swapped),
    "s04_truncation": lambda: _mutant(
        quantize_groups=lambda w, g, symmetric=False: _quantize_variant(w, g, symmetric, rnd=np.trunc)),
    "s07_f32_quotient_against_stored_scale": lambda: _mutant(
        quantize_groups=lambda w, g, symmetric=False: _quantize_variant(w, g, symmetric, f32_quotient=True)),
    "s08_scale_range_over_16": lambda: _mutant(
        quantize_groups=lambda w, g, symmetric=False: _quantize_variant(w, g, symmetric, qden_scale=16)),
    "zero_added_before_rounding": lambda: _mutant(
        quantize_groups=lambda w, g, symmetric=False: _quantize_variant(w, g, symmetric, zero_inside=True)),
    "s10_odd_group_accepted": lambda: _mutant(dequantize_int4_groups=_dequant_odd_ok),
    "s16_bias_dropped": lambda: _mutant(
        linear_int4_groups=lambda *a, **kw: _linear_variant(*a, drop_bias=True, **kw)),
    "s17_w_not_transposed": lambda: _mutant(
        linear_int4_groups=lambda *a, **kw: _linear_variant(*a, transpose_w=True, **kw)),
    "m01_scales_on_wrong_axis": lambda: _mutant(
        linear_int4_groups=lambda *a, **kw: _linear_variant(*a, wrong_axis=True, **kw)),
    "order_scatter_not_gather": lambda: _mutant(
        linear_int4_groups=lambda *a, **kw: _linear_variant(*a, scatter=True, **kw)),
    "bf16_truncation": lambda: _mutant(
        bf16_round_bits=lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)),
    "rint_half_away": lambda: _mutant(rint_half_even=lambda a: np.trunc(np.asarray(a) + np.copysign(0.5, a))),
    "prepare_rows_and_quarters_swapped": lambda: _mutant(
        prepare_int4=lambda p, n, k: _prepare_variant(p, n, k, swap_lanes=True)),
    "prepare_step_major_blocks": lambda: _mutant(
        prepare_int4=lambda p, n, k: _prepare_variant(p, n, k, step_major=True)),
    "prepare_pads_with_ones": lambda: _mutant(
        prepare_int4=lambda p, n, k: _prepare_variant(p, n, k, pad=0xFF)),
    "unprepare_drops_last_tile": lambda: _mutant(
        unprepare_int4=lambda pr, n, k: oracle.unprepare_int4(pr, n, k)[: max(n - 1, 0) or n]),
}


def _prepare_variant(p, n, k, swap_lanes=False, step_major=False, pad=0):
    if k % 32:
        raise ValueError("bad")
    nt, ns = -(-n // 16), -(-k // 128)
    rows = np.full((nt * 16, ns * 64), pad, dtype=np.uint8)
    rows[:n, :k // 2] = np.asarray(p, dtype=np.uint8).reshape(n, k // 2)
    b = rows.reshape(nt, 16, ns, 4, 16)
    order = (0, 2, 1, 3, 4) if swap_lanes else (0, 2, 3, 1, 4)
    if step_major:
        order = (2, 0, 3, 1, 4)
    return np.ascontiguousarray(b.transpose(order)).reshape(-1)


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


# ---------------------------------------------------------------------------
# Property test over random groups (the oracle only)
# ---------------------------------------------------------------------------

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=60, deadline=None)
@given(group=st.sampled_from([2, 16, 32, 64, 128, 256]),
       log_scale=st.floats(min_value=-3, max_value=2),
       seed=st.integers(min_value=0, max_value=2 ** 31 - 1),
       skew=st.floats(min_value=-0.9, max_value=0.9))
def test_half_step_bound_property(group, log_scale, seed, skew):
    rng = np.random.default_rng(seed)
    w = ((rng.standard_normal((4, 2 * group)) + skew) * 10.0 ** log_scale).astype(np.float32)
    ok, _, _ = _half_step_ok(oracle_impl(), w, group)
    assert ok
