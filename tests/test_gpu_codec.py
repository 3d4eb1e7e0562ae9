"""GPU quantize / pack / unpack / dequantize against the CPU oracle: bit-exact."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import load_golden, parse_nums

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _quant_both(woq, w, group, symmetric=False):
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group, symmetric)
    qr, sr, zr = oracle.quantize_groups(w, group, symmetric)
    return (q.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy()), (qr, sr, zr)


def _assert_same(gpu, ref, what):
    for a, b, name in zip(gpu, ref, ("q", "scale", "zero")):
        if name == "scale":
            ok = np.array_equal(a.view(np.uint32), b.view(np.uint32))
        else:
            ok = np.array_equal(a, b)
        if not ok:
            bad = np.argwhere(a.view(np.uint32) != b.view(np.uint32)) if name == "scale" else np.argwhere(a != b)
            raise AssertionError(f"{what}: {name} differs at {bad[:5].tolist()} ({len(bad)} places)")


@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("symmetric", [False, True])
def test_quantize_random_bit_exact(woq, group, symmetric):
    _say(f"quantize random group={group} symmetric={symmetric}")
    w = workloads.weight(37, 4 * group, seed=group + 7, std=0.02)
    w[3] = 0.0                                  # all-zero row
    w[4, :group] = np.float32(0.125)            # constant group
    w[5, :group] = np.linspace(-1, 14, group, dtype=np.float32)   # many exact ties
    w[6] *= np.float32(1e-38 / 0.02)           # subnormal range
    gpu, ref = _quant_both(woq, w, group, symmetric)
    _assert_same(gpu, ref, f"group {group}")


def test_quantize_tiny_config_and_odd_groups(woq):
    c = workloads.TINY
    w = workloads.weight(c.n, c.k, c.seed_w)
    _assert_same(*_quant_both(woq, w, c.group), "tiny")
    for group, shape in ((5, (3, 20)), (6, (4, 18)), (2, (2, 8)), (12, (5, 36))):
        w = workloads.weight(*shape, seed=group, std=1.0)
        _assert_same(*_quant_both(woq, w, group), f"group {group}")
        _assert_same(*_quant_both(woq, w, group, True), f"group {group} symmetric")


def test_quantize_worked_examples(woq):
    g = load_golden("symmetric_int4_group5.txt")
    w = np.array([[float(v) for v in parse_nums(g["w"])]], dtype=np.float32)
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), 5, symmetric=True)
    assert (q.cpu().numpy().astype(int) - 8).tolist() == [[int(v) for v in parse_nums(g["codes"])]]
    g = load_golden("symmetric_int4_group4_rows.txt")
    w = np.array([[float(v) for v in parse_nums(g["row0_w"])],
                  [float(v) for v in parse_nums(g["row1_w"])]], dtype=np.float32)
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), 4, symmetric=True)
    codes = q.cpu().numpy().astype(int) - 8
    assert codes[0].tolist() == [int(v) for v in parse_nums(g["row0_codes"])]
    assert codes[1].tolist() == [int(v) for v in parse_nums(g["row1_codes"])]
    nib = torch.from_numpy((codes & 0xF).astype(np.uint8)).cuda()
    packed = woq.pack_uint4(nib).cpu().numpy()
    assert packed[0].tolist() == [int(t, 16) for t in g["row0_bytes_hex"].split()]
    assert packed[1].tolist() == [int(t, 16) for t in g["row1_bytes_hex"].split()]


def test_quantize_rejects_non_finite(woq):
    w = np.zeros((4, 64), dtype=np.float32)
    for bad in (np.nan, np.inf, -np.inf):
        w[2, 17] = bad
        with pytest.raises(woq.WoqError) as e:
            woq.quantize_groups(torch.from_numpy(w).cuda(), 32)
        assert e.value.name == "WOQ_ENONFINITE"


def test_pack_unpack_exhaustive_and_errors(woq):
    lo, hi = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    pairs = np.stack([lo.ravel(), hi.ravel()], -1).astype(np.uint8)
    for arr in (pairs, pairs.reshape(1, 512), np.ascontiguousarray(pairs[:128])):
        g = woq.pack_uint4(torch.from_numpy(arr).cuda()).cpu().numpy()
        assert np.array_equal(g, oracle.pack_uint4(arr))
    allb = np.arange(256, dtype=np.uint8)
    for arr in (allb, allb.reshape(16, 16), allb[:8]):
        g = woq.unpack_uint4(torch.from_numpy(np.ascontiguousarray(arr)).cuda()).cpu().numpy()
        assert np.array_equal(g, oracle.unpack_uint4(arr))
    bad = pairs.copy()
    bad[77, 1] = 16
    with pytest.raises(woq.WoqError) as e:
        woq.pack_uint4(torch.from_numpy(bad).cuda())
    assert e.value.name == "WOQ_ERANGE"
    # unaligned start (odd byte offset) takes the byte-wise kernels
    base = torch.from_numpy(np.concatenate([[0], pairs.ravel()]).astype(np.uint8)).cuda()
    view = base[1:]
    lib = woq.load()
    out = torch.empty(256, dtype=torch.uint8, device="cuda")
    assert lib.woq_pack_uint4(view.data_ptr(), 512, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.pack_uint4(pairs).ravel())


def test_pack_unpack_large_random(woq):
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, (1000, 4096), dtype=np.uint8)
    p = woq.pack_uint4(torch.from_numpy(q).cuda())
    assert np.array_equal(p.cpu().numpy(), oracle.pack_uint4(q))
    assert np.array_equal(woq.unpack_uint4(p).cpu().numpy(), q)


@pytest.mark.parametrize("group", [4, 6, 32, 64, 128, 256])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bit_exact(woq, group, out):
    rng = np.random.default_rng(group)
    n, k = 33, group * 6
    q = rng.integers(0, 16, (n, k), dtype=np.uint8)
    s = (rng.standard_normal((n, k // group)) * 0.01).astype(np.float32)
    s[0, 0] = np.float32(3.3e-39)
    s[1, 0] = np.float32(3.0e38)
    z = rng.integers(0, 16, (n, k // group), dtype=np.uint8)
    packed = oracle.pack_uint4(q)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    g = woq.dequantize_int4_groups(torch.from_numpy(packed).cuda(), torch.from_numpy(s).cuda(),
                                   torch.from_numpy(z).cuda(), group, dt)
    ref = oracle.dequantize_int4_groups(packed, s, z, n, k, group, out)
    if out == "f32":
        assert np.array_equal(g.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    else:
        assert np.array_equal(g.view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.slow
@pytest.mark.parametrize("n,k", [(14336, 4096), (28672, 8192)])
def test_quantize_full_size_bit_exact(woq, n, k):
    _say(f"quantize full size {n}x{k}")
    w = workloads.weight(n, k, seed=140, outlier_frac=0.01, seed_cols=540)
    q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), 128)
    packed = woq.pack_uint4(q)
    qr, sr, zr = oracle.quantize_groups(w, 128)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(z.cpu().numpy(), zr)
    assert np.array_equal(packed.cpu().numpy(), oracle.pack_uint4(qr))
