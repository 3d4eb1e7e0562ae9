"""The quantizers' outputs through the linear layer on the GPU.

GPTQ ("20. Quantization", stretch exercise 4; linnet "Importing GPTQ and AWQ":
in activation order the layer gathers its inputs through `order`) and AWQ
(stretch exercise 3, with the page's identity X W^T = (X S^-1)(W S)^T: the
scaled layer takes x / s).  Each packs into the Int4GroupLinear layout and
runs through woq_linear_int4_groups; the results match the oracle's linear on
the same tensors to the linear layer's bar, and on held-out inputs drawn from
the calibration set's distribution both beat round to nearest against the
unquantized layer.  Each case prints its name
first.
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


def _rel_err(y, y_true):
    return float(np.linalg.norm(y - y_true) / np.linalg.norm(y_true))


@pytest.mark.parametrize("m", [1, 16, 200])
def test_gptq_act_order_through_the_linear(woq, m):
    n, k, t, group = 512, 1024, 256, 128
    _say(f"gptq -> linear m={m} n={n} k={k} act_order")
    w = workloads.weight(n, k, seed=41)
    x_all = workloads.calibration_bf16(t + m, k, seed=42)   # one distribution: calibration rows, then held-out rows
    xc, x = x_all[:t], np.ascontiguousarray(x_all[t:])
    wd = torch.from_numpy(w).cuda()
    q, sc, z, order = woq.gptq_quantize(wd, to_dev_bf16(xc), group, act_order=True)
    packed = woq.pack_uint4(q)
    y = woq.linear_int4_groups(to_dev_bf16(x), packed, sc, z, order=order, group=group, out_dtype=torch.float32)
    qr, sr, zr = woq.quantize_groups(wd, group)
    y_rtn = woq.linear_int4_groups(to_dev_bf16(x), woq.pack_uint4(qr), sr, zr, group=group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref = oracle.linear_int4_groups(x, packed.cpu().numpy(), sc.cpu().numpy(), z.cpu().numpy(), n, k, group,
                                      order=order.cpu().numpy())
    check_linear(y, y_ref, f"gptq m={m}")
    y_true = oracle.bf16_bits_to_f64(x) @ w.astype(np.float64).T
    e_gptq, e_rtn = _rel_err(y.cpu().numpy(), y_true), _rel_err(y_rtn.cpu().numpy(), y_true)
    _say(f"  relative output error: gptq {e_gptq:.4f}, round to nearest {e_rtn:.4f}")
    assert e_gptq < e_rtn


@pytest.mark.parametrize("m", [1, 64])
def test_awq_scaled_layer_through_the_linear(woq, m):
    n, k, t, group = 384, 1024, 128, 128
    _say(f"awq -> linear m={m} n={n} k={k}")
    w = workloads.weight(n, k, seed=51)
    x_all = workloads.calibration_bf16(t + m, k, seed=52, channel_spread=1.5)
    xc, x = x_all[:t], np.ascontiguousarray(x_all[t:])
    wd = torch.from_numpy(w).cuda()
    q, sc, z, s, best, _ = woq.awq_search(wd, to_dev_bf16(xc), group)
    assert best > 0
    xs = (to_dev_bf16(x).float() / s).to(torch.bfloat16)      # the caller's x S^-1, rounded to bf16
    packed = woq.pack_uint4(q)
    y = woq.linear_int4_groups(xs, packed, sc, z, group=group, out_dtype=torch.float32)
    qr, sr, zr = woq.quantize_groups(wd, group)
    y_rtn = woq.linear_int4_groups(to_dev_bf16(x), woq.pack_uint4(qr), sr, zr, group=group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    xs_bits = xs.view(torch.int16).cpu().numpy().view(np.uint16)
    check_linear(y, oracle.linear_int4_groups(xs_bits, packed.cpu().numpy(), sc.cpu().numpy(), z.cpu().numpy(),
                                              n, k, group), f"awq m={m}")
    y_true = oracle.bf16_bits_to_f64(x) @ w.astype(np.float64).T
    e_awq, e_rtn = _rel_err(y.cpu().numpy(), y_true), _rel_err(y_rtn.cpu().numpy(), y_true)
    _say(f"  relative output error: awq {e_awq:.4f}, round to nearest {e_rtn:.4f}")
    assert e_awq < e_rtn
