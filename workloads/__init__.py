"""Seeded synthetic inputs for the group-wise 4-bit linear layer.

This module only draws random numbers and names shapes.  It holds none of the
method's arithmetic (no quantization, packing, dequantization or products), so
the CPU oracle and the HIP library can both be fed from it without sharing any
of the computation they are checked on.

Shapes and distributions follow the Llama-3-8B-shaped workloads used to
measure the layer (decode GEMVs, a small-M sweep, prefill GEMMs and an
act-order case).  The pages measure on Llama 3.1 8B decode and on a
perplexity dataset; no model weights or dataset exist here, so these seeded
Gaussian tensors of the same shapes stand in for them.

Every generator uses ``numpy.random.default_rng(seed)`` (PCG64), so a given
seed yields the same bytes on any host.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "LinearCase",
    "weight",
    "activations_bf16",
    "bias",
    "order",
    "order_with_repeats",
    "bf16_bits_to_f32",
    "TINY",
    "DECODE",
    "SWEEP",
    "PREFILL",
    "ACTORDER",
    "SYM16",
    "ZP4",
    "MXFP4",
    "LLAMA3_8B_LAYER",
    "MIDSIZE",
    "SMALLBATCH",
    "FEWROWS",
]


@dataclass(frozen=True)
class LinearCase:
    """One linear-layer workload: y[M,N] = x[M,K] . W[N,K]^T (+ bias)."""

    name: str
    m: int
    n: int
    k: int
    group: int = 128
    has_bias: bool = False
    act_order: bool = False
    outlier_frac: float = 0.0
    seed_w: int = 0
    seed_x: int = 0
    seed_bias: int = 0
    seed_order: int = 0
    seed_cols: int = 0
    tags: tuple = field(default_factory=tuple)


def weight(n: int, k: int, seed: int, std: float = 0.02,
           outlier_frac: float = 0.0, outlier_mult: float = 20.0,
           seed_cols: int = 0) -> np.ndarray:
    """W ~ N(0, std^2) as float32 [n, k].

    With ``outlier_frac > 0``, ``round(outlier_frac * k)`` distinct columns
    (drawn with ``seed_cols``) are multiplied by ``outlier_mult``: the
    act-order workload's salient input channels, in stored column order.
    """
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    if outlier_frac > 0:
        cnt = int(round(outlier_frac * k))
        cols = np.random.default_rng(seed_cols).choice(k, size=cnt, replace=False)
        w[:, cols] *= np.float32(outlier_mult)
    return w


def activations_bf16(m: int, k: int, seed: int, outlier_frac: float = 0.0, outlier_mult: float = 50.0,
                     offset: float = 0.0, seed_cols: int = 0) -> np.ndarray:
    """x ~ N(0, 1) (+ offset) rounded to bfloat16; returned as raw uint16 bit patterns [m, k].

    With ``outlier_frac > 0``, ``round(outlier_frac * k)`` distinct input
    channels (drawn with ``seed_cols``) are multiplied by ``outlier_mult``: a
    few salient activation channels, the premise of activation-aware scaling.
    ``offset`` is added to every entry (a large common mean).
    """
    import torch

    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((m, k), dtype=np.float32)
    if outlier_frac > 0:
        cnt = int(round(outlier_frac * k))
        cols = np.random.default_rng(seed_cols).choice(k, size=cnt, replace=False)
        x32[:, cols] *= np.float32(outlier_mult)
    if offset:
        x32 += np.float32(offset)
    xb = torch.from_numpy(x32).to(torch.bfloat16)
    return xb.view(torch.int16).numpy().view(np.uint16).copy()


def calibration_bf16(t: int, k: int, seed: int, rank: int = 16, noise: float = 0.3,
                     channel_spread: float = 0.5) -> np.ndarray:
    """Calibration activations for GPTQ: correlated input channels (a rank-`rank`
    mix of N(0, 1) factors plus N(0, noise^2) per entry) with a log-normal
    magnitude per channel (sigma `channel_spread`), rounded to bfloat16; raw
    uint16 bit patterns [t, k]."""
    import torch

    rng = np.random.default_rng(seed)
    mix = rng.standard_normal((t, rank)) @ rng.standard_normal((rank, k)) / np.sqrt(rank)
    x = (mix + noise * rng.standard_normal((t, k))) * np.exp(channel_spread * rng.standard_normal(k))
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    return xb.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns to float32 (exact: a bit shift)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bias(n: int, seed: int, std: float = 0.01) -> np.ndarray:
    """bias ~ N(0, std^2) as float32 [n]."""
    rng = np.random.default_rng(seed)
    b = rng.standard_normal(n, dtype=np.float32)
    b *= np.float32(std)
    return b


def order(k: int, seed: int) -> np.ndarray:
    """A seeded random permutation of range(k) as int32: the act-order gather index."""
    return np.random.default_rng(seed).permutation(k).astype(np.int32)


def order_with_repeats(k: int, seed: int) -> np.ndarray:
    """k gather indices drawn uniformly from range(k) with replacement (int32):
    in range but not a permutation, so some inputs repeat and others are skipped."""
    return np.random.default_rng(seed).integers(0, k, size=k).astype(np.int32)


# ---------------------------------------------------------------------------
# Workload registry (seeds are fixed so every run draws identical tensors)
# ---------------------------------------------------------------------------

TINY = LinearCase("tiny_1x64x256_g32", m=1, n=64, k=256, group=32,
                  seed_w=101, seed_x=201)

# Llama-3-8B decode GEMVs at M=1, group 128; the first (4096x4096) carries a bias.
DECODE = (
    LinearCase("decode_q_4096x4096", 1, 4096, 4096, 128, has_bias=True,
               seed_w=110, seed_x=210, seed_bias=310),
    LinearCase("decode_kv_1024x4096", 1, 1024, 4096, 128, seed_w=111, seed_x=211),
    LinearCase("decode_gateup_14336x4096", 1, 14336, 4096, 128, seed_w=112, seed_x=212),
    LinearCase("decode_down_4096x14336", 1, 4096, 14336, 128, seed_w=113, seed_x=213),
)

_SWEEP_GSEED = {32: 0, 64: 1, 128: 2, 256: 3}
SWEEP = tuple(
    LinearCase(f"sweep_m{m}_g{g}_14336x4096", m, 14336, 4096, g,
               seed_w=120 + _SWEEP_GSEED[g], seed_x=220 + m)
    for g in (32, 64, 128, 256) for m in (1, 4, 16, 64, 128)
)

PREFILL = (
    LinearCase("prefill_2048_14336x4096", 2048, 14336, 4096, 128, seed_w=130, seed_x=230),
    LinearCase("prefill_2048_4096x14336", 2048, 4096, 14336, 128, seed_w=131, seed_x=231),
)

ACTORDER = tuple(
    LinearCase(f"actorder_m{m}_{n}x{k}", m, n, k, 128, has_bias=True, act_order=True,
               outlier_frac=0.01, seed_w=140 + i, seed_x=240 + i + 10 * j,
               seed_bias=340 + i, seed_order=440 + i, seed_cols=540 + i)
    for i, (n, k) in enumerate(((28672, 8192), (8192, 28672)))
    for j, m in enumerate((1, 16))
)

# The seven quantized linears of one Llama-3-8B decoder layer (hidden 4096,
# 8 KV heads of 128, MLP 14336), in execution order.  The q projection
# carries the one bias of the decode workload.
LLAMA3_8B_LAYER = (
    ("q", 4096, 4096, True),
    ("k", 1024, 4096, False),
    ("v", 1024, 4096, False),
    ("o", 4096, 4096, False),
    ("gate", 14336, 4096, False),
    ("up", 14336, 4096, False),
    ("down", 4096, 14336, False),
)
LLAMA3_8B_LAYERS = 32


def packed_weights(n: int, k: int, group: int, seed: int, std: float = 0.02):
    """Int4GroupLinear tensors drawn directly at random (no quantizer involved).

    packed: uniform bytes [n, k/2]; scale: float32 [n, k/group] with the
    magnitude a 4-bit grid over N(0, std^2) groups has (|N(0,1)|*std*4/15 +
    std/15); zero: uniform 0..15.  Used where only the layout and size of a
    quantized weight matter (timing the CPU oracle on a bounded sample).
    """
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scale = (np.abs(rng.standard_normal((n, k // group))) * std * 4 / 15 + std / 15).astype(np.float32)
    zero = rng.integers(0, 16, (n, k // group), dtype=np.uint8)
    return packed, scale, zero


# Signed int4 groups with float16 scales (tinyllm L8.5, "int4 per group", whose
# default group is 32): the decode shapes at M = 1 with groups 32 and 128,
# one small-M and one prefill shape.
# Batches between the small-M kernel and prefill on the same Llama-3-8B
# shapes (the tiled GEMM, split over K on the narrow layers): sizes only, no
# figure from the pages.
MIDSIZE = tuple(
    LinearCase(f"midsize_m{m}_{n}x{k}", m, n, k, 128, seed_w=180 + i, seed_x=280 + i + 10 * j)
    for j, m in enumerate((128, 256))
    for i, (n, k) in enumerate(((1024, 4096), (4096, 4096), (4096, 14336), (14336, 4096)))
)

# Small batches (16 and 64 rows) on the same Llama-3-8B shapes: the layers
# narrower than 800 tiles of 16 rows run on the small-M path with the
# activation slice in LDS, 14336x4096 on the small-M kernel.  Sizes only, no
# figure from the pages.
SMALLBATCH = tuple(
    LinearCase(f"smallbatch_m{m}_{n}x{k}", m, n, k, 128, seed_w=185 + i, seed_x=285 + i + 10 * j)
    for j, m in enumerate((16, 64))
    for i, (n, k) in enumerate(((1024, 4096), (4096, 4096), (4096, 14336), (14336, 4096)))
)

# Two to four activation rows (a few decode streams at once) on the same
# Llama-3-8B shapes and on 8192x28672: the row-streaming kernel, or the tile
# GEMV on the layers of at least 2^25 weights with K >= 8192.  Sizes only, no
# figure from the pages.
FEWROWS = tuple(
    [LinearCase(f"fewrows_m{m}_{n}x{k}", m, n, k, 128, seed_w=190 + i, seed_x=290 + i + 10 * j)
     for j, m in enumerate((2, 3, 4))
     for i, (n, k) in enumerate(((1024, 4096), (4096, 4096), (4096, 14336), (14336, 4096)))]
    + [LinearCase(f"fewrows_m{m}_8192x28672", m, 8192, 28672, 128, seed_w=195, seed_x=295 + m) for m in (2, 4)]
)

SYM16 = tuple(
    [LinearCase(f"sym16_m1_g{g}_{n}x{k}", 1, n, k, g, seed_w=150 + i, seed_x=250 + i)
     for g in (32, 128) for i, (n, k) in enumerate(((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)))]
    + [LinearCase("sym16_m16_g32_14336x4096", 16, 14336, 4096, 32, seed_w=158, seed_x=258),
       LinearCase("sym16_m2048_g32_4096x14336", 2048, 4096, 14336, 32, seed_w=159, seed_x=259)]
)


# Packed 4-bit zero points (the MatMulNBits layout): the g128 decode, small-M
# and prefill shapes, timed per call (the unpack into the workspace included).
ZP4 = tuple(
    [LinearCase(f"zp4_m1_g128_{n}x{k}", 1, n, k, 128, seed_w=170 + i, seed_x=270 + i)
     for i, (n, k) in enumerate(((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)))]
    + [LinearCase("zp4_m16_g128_14336x4096", 16, 14336, 4096, 128, seed_w=174, seed_x=274),
       LinearCase("zp4_m2048_g128_14336x4096", 2048, 14336, 4096, 128, seed_w=175, seed_x=275)]
)


# MXFP4 (linnet "MXFP4 experts"; blocks of 32 with an E8M0 scale): the same
# decode, small-M and prefill shapes.
MXFP4 = tuple(
    [LinearCase(f"mxfp4_m1_{n}x{k}", 1, n, k, 32, seed_w=160 + i, seed_x=260 + i)
     for i, (n, k) in enumerate(((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)))]
    + [LinearCase("mxfp4_m16_14336x4096", 16, 14336, 4096, 32, seed_w=164, seed_x=264),
       LinearCase("mxfp4_m2048_14336x4096", 2048, 14336, 4096, 32, seed_w=165, seed_x=265),
       LinearCase("mxfp4_m2048_4096x14336", 2048, 4096, 14336, 32, seed_w=166, seed_x=266)]
)

