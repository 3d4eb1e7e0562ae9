"""GPU: several linears over the same activations in one call
(woq_linear_int4_groups_grouped) against the float64 oracle and against the
separate calls.  Each case prints its name before it touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_linear, to_dev_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _mats(woq, ns, k, group, seed, biases):
    out = []
    for i, n in enumerate(ns):
        w = workloads.weight(n, k, seed=seed + 10 * i)
        b = workloads.bias(n, seed=seed + 10 * i + 3) if biases[i] else None
        q, s, z = woq.quantize_groups(torch.from_numpy(w).cuda(), group)
        out.append(dict(w=w, b=b, packed=woq.pack_uint4(q), scale=s, zero=z,
                        bias=None if b is None else torch.from_numpy(b).cuda()))
    return out


def _ref(x, mat, group, k):
    qr, sr, zr = oracle.quantize_groups(mat["w"], group)
    return oracle.linear_int4_groups(x, oracle.pack_uint4(qr), sr, zr, mat["w"].shape[0], k, group,
                                     bias=mat["b"])


CASES = [
    # m, row counts, k, group, which matrices have a bias
    (1, (48, 17, 100), 1024, 128, (True, False, True)),   # ragged tiles, one launch
    (1, (64, 64), 4096, 32, (False, False)),
    (2, (30, 50, 70, 16), 768, 64, (False, True, False, True)),
    (4, (100, 33), 2048, 256, (True, True)),
    (8, (48, 80), 1024, 128, (True, False)),             # small-M path: one call per matrix
    (40, (64, 20), 512, 64, (False, True)),              # tiled GEMM path
    (1, (0, 33), 512, 128, (False, True)),               # an empty matrix
]


@pytest.mark.parametrize("m,ns,k,group,biases", CASES)
@pytest.mark.parametrize("prepared", [False, True])
def test_grouped_matches_oracle_and_separate_calls(woq, m, ns, k, group, biases, prepared):
    _say(f"grouped m={m} n={ns} k={k} g={group} prepared={prepared} "
         f"plan(total rows): {woq.linear_plan(m, sum(ns), k, group)}")
    x = workloads.activations_bf16(m, k, seed=900 + m + k)
    xd = to_dev_bf16(x)
    mats = _mats(woq, ns, k, group, seed=700 + m, biases=biases)
    weights = [woq.prepare_int4(d["packed"], k) if prepared else d["packed"] for d in mats]
    args = [(wt, d["scale"], d["zero"], d["bias"]) for wt, d in zip(weights, mats)]
    for out in (torch.float32, torch.bfloat16):
        ys = woq.linear_int4_groups_grouped(xd, args, prepared=prepared, out_dtype=out)
        torch.cuda.synchronize()
        for i, (d, y) in enumerate(zip(mats, ys)):
            assert tuple(y.shape) == (m, ns[i])
            if ns[i] == 0:
                continue
            check_linear(y, _ref(x, d, group, k), f"grouped matrix {i} out={out}")
            single = woq.linear_int4_groups(xd, d["packed"], d["scale"], d["zero"], bias=d["bias"],
                                            group=group, out_dtype=torch.float32)
            torch.cuda.synchronize()
            if out == torch.float32:
                diff = (y - single).abs().max().item()
                scale = single.abs().max().item()
                assert diff <= 1e-5 * scale, f"matrix {i}: grouped vs separate {diff:.3e} (max |y| {scale:.3e})"


@pytest.mark.slow
def test_grouped_llama_qkv_and_gate_up(woq):
    """The decode projections that share an input, at full size, against the
    separate calls (whose full-size parity the linear tests establish) and the
    oracle on sampled rows."""
    for ns, k in (((4096, 1024, 1024), 4096), ((14336, 14336), 4096)):
        _say(f"grouped full size n={ns} k={k}")
        x = workloads.activations_bf16(1, k, seed=31)
        xd = to_dev_bf16(x)
        mats = _mats(woq, ns, k, 128, seed=41, biases=(True,) + (False,) * (len(ns) - 1))
        ys = woq.linear_int4_groups_grouped(xd, [(d["packed"], d["scale"], d["zero"], d["bias"]) for d in mats],
                                            out_dtype=torch.float32)
        torch.cuda.synchronize()
        rng = np.random.default_rng(5)
        for i, (d, y) in enumerate(zip(mats, ys)):
            single = woq.linear_int4_groups(xd, d["packed"], d["scale"], d["zero"], bias=d["bias"],
                                            group=128, out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert (y - single).abs().max().item() <= 1e-5 * single.abs().max().item()
            rows = np.unique(np.concatenate([[0, ns[i] - 1], rng.choice(ns[i], 24, replace=False)]))
            sub = dict(w=d["w"][rows], b=None if d["b"] is None else d["b"][rows])
            check_linear(y[:, torch.from_numpy(rows).cuda()], _ref(x, sub, 128, k), f"full grouped {i}")
