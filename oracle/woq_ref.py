"""CPU oracle for the group-wise 4-bit weight-only linear layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This module is the yardstick the HIP
library is measured against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code,
tables or constants with the HIP library, and never calls it.

Everything is plain NumPy, evaluated in float64, written to be checked against
the pages by eye.  Sources (page title, then section):

* linnet docs, "Quantization": the std.quant table (the Int4GroupLinear layout
  ``weight [Out, In/Group, Group/2; u8]``, scale and zero ``[Out, In/Group]``,
  optional ``order [In; i32]`` and bias; ``dequantize_int4_groups`` computes
  ``(q - zero) * scale`` per group; ``linear_int4_groups`` is a linear layer
  over those weights), the sentence on packed 4-bit formats (two values per
  byte, even element in the low nibble), section "Group-wise 4-bit weights"
  (16 levels per group with a scale and a zero point) and section "Importing
  GPTQ and AWQ" (an act-order layer gathers its inputs through ``order``).
* tinyllm L8.5, "Quantization: int8, int4 group (packed), fp8, KV quant":
  section 2 "Principles" (symmetric scaling, ties-to-even rounding, the
  half-step bound, packing), section 3 "Worked example by hand".
* "20. Quantization" (inference book): section "Symmetric quantization, from
  scratch" (s = a/Q, codes clamp(round(w/s)), worked example), the edge case
  of an all-zero group getting scale 1, section "Packing".
* "4.8 Quantization II": section "The Quantization Landscape: A Taxonomy"
  (asymmetric scheme with a zero point; half-step bound; s^2/12 noise) and
  section "Per-Group INT4" (unsigned codes [0, 15] with a zero point).

Readings taken where the pages are silent or disagree (each is listed with
its reason in the design notes of the repository):

R1  The rounding step rounds the *real* quotient ``Q*w/range`` to the nearest
    integer, ties to even, evaluated as one float64 division of float64
    operands.  This reproduces the inference book's worked example
    ``[-2,-1,0,1,2] -> [-7,-4,0,4,7]``; forming the quotient in float32
    against the stored scale would give ``[-7,-3,0,3,7]`` there.
R2  Asymmetric scheme: ``range = max - min`` of the raw group (not widened to
    include 0); ``scale = f32(range/15)``; ``zero = clamp(rint(-15*min/range),
    0, 15)``; ``q = clamp(rint(15*w/range) + zero, 0, 15)``.  The rounding is
    applied to ``w/scale`` before the zero point is added.
R3  A group with range 0 gets scale 1 (the inference book's rule for an
    all-zero group, extended to any constant group): ``zero = clamp(rint(-min),
    0, 15)``, ``q = clamp(rint(w) + zero, 0, 15)``.
R4  Symmetric scheme (worked-example mode): ``a = max|w|``; ``scale =
    f32(a/7)``; ``c = clamp(rint(7*w/a), -7, 7)``; stored unsigned as
    ``q = c + 8`` with ``zero = 8``, so ``(q - zero)*scale = c*scale``.  An
    all-zero group gets scale 1 and c = 0.
R5  Scale is stored as float32 and zero as uint8.
R6  ``order`` is a gather: ``x'[m, k] = x[m, order[k]]``.
R7  Dequantization forms ``(q - zero) * scale`` once, rounded to float32, and
    then (for a bfloat16 result) rounds that float32 to bfloat16.
R8  The linear layer's exact value is ``sum_k x'[m,k] * (q-z)*s + bias[n]``
    with the float64-exact ``(q - z)*s`` (a 4-bit integer times a float32 is
    exact in float64).
R9  Prepared weights.  The linnet page says its fused int4 kernels run on
    weights re-ordered once at load time ("--prepare") and the inference book
    names a kernel-specific re-ordering, but neither gives the order.  The
    order used here is this library's own: blocks of 16 outputs x 128 inputs
    (1024 bytes), tile-major then step-major; inside a block, lane slot l
    (16 bytes) holds output row 16t + l % 16, packed bytes
    [64 s + 16 (l // 16), +16) of that row, i.e. inputs 128 s + 32 (l // 16)
    .. +32.  Rows past N and bytes past K/2 are zero.  Scale and zero keep the
    canonical layout.  The linear layer over prepared weights has the value
    of R8 over the canonical weights they came from.
R10 Signed int4 groups with float16 scales (tinyllm L8.5, section 2, "int4
    per group" and "Packing"): per group of G inputs, ``s16 =
    float16(amax / 7)`` with the quotient formed in float32 (the page forms
    every quotient in float32) and then rounded once more, to float16,
    ties to even; codes ``c = clamp(rint(float32(w / s16)), -8, 7)``, the
    quotient again in float32, against the stored float16 value.  A group
    whose s16 is 0 (all zero, or amax / 7 below float16's range) gets codes 0
    and scale 0; an s16 that overflows float16 is refused.  Bytes hold two
    4-bit two's complement codes, the even input in the low nibble.
    ``dequant = c * s16`` (exact in float32), and the linear layer's exact
    value is ``sum_k x'[m,k] * c * s16 + bias[n]`` as in R8.
R11 MXFP4 (linnet "Quantization", std.quant table, dequantize_mxfp4: E2M1
    values in blocks of 32, one E8M0 scale byte a block; tinyllm L8.5 section
    2, "MXFP4": a block's power-of-two scale X, elements 0, 0.5, 1, 1.5, 2, 3,
    4, 6 times X, values above 6X saturate, every element within 2X).  Layout:
    blocks [N, K/32, 16] uint8, two 4-bit E2M1 codes a byte, the even element
    in the low nibble (linnet packing sentence); scales [N, K/32] uint8, X =
    2^(e - 127).  Code c: bit 3 the sign, bits 0..2 index the magnitudes
    above.  The pages do not say how X is chosen; the reading follows the OCP
    Microscaling Formats v1.0 rule the page cites for depth: X = 2^(floor(
    log2 amax) - 2) (2 = the largest E2M1 exponent), e = clamp(floor(log2
    amax) - 2 + 127, 0, 254), e = 0 for a zero block.  Elements round w / X
    (exact) to the nearest magnitude, ties to the even code, saturate at 6,
    and keep their sign (a negative value that rounds to 0 is code 8).
    ``dequant = code_value * X`` (exact in float32); the linear layer's exact
    value is ``sum_k x[m,k] * dequant[n,k] + bias[n]``.
R12 Int4Linear (linnet "Quantization", std.quant table: weight [Out, In/2]
    of two signed nibbles a byte, the even element low; one float32 scale a
    row, as the page's Mlp example declares; dequantize_int4 = unpack, then
    dequantize).  The page gives the layout, not the quantizer; the rule is
    tinyllm L8.5's symmetric scaling (section 2) with q_max = 7 and one scale
    per row: s = float32(amax / 7) (a float32 quotient), codes
    c = clamp(rint(float32(w / s)), -8, 7), a zero row gets s = 0 and codes 0.
    ``dequant = c * s`` rounded once to float32; the linear layer's exact value
    is ``sum_k x'[m,k] * c * s + bias[n]`` with the float64-exact c * s.
R13 GPTQ ("20. Quantization", stretch exercise 4: accumulate H = 2 X^T X
    from calibration inputs, quantize column by column, spreading each
    column's error over the remaining columns with the Cholesky factor of
    H^-1; linnet "Importing GPTQ and AWQ": in activation order the layer
    gets an `order` and gathers its inputs).  The steps not printed there
    follow the published method (Frantar et al., GPTQ): columns with
    H_jj = 0 are zeroed and get H_jj = 1; with act_order the columns are
    visited by decreasing H_jj (a stable sort) and `order` is that
    permutation; H += damp * mean(diag H) * I; U is the upper Cholesky
    factor of H^-1; for each column i, at the first column of each group
    the group's scale and zero come from its current (already updated)
    columns by R2, the column is coded by R2, and with
    err = (w_i - dequant_i) / U_ii every later column j takes
    w_j -= err * U_ij.  The factor 2 in H and its normalisation do not
    change U's use (it scales U and err inversely), so H = X^T X here.
R14 AWQ ("20. Quantization", stretch exercise 3: for one linear layer, a
    per-input-channel scale s_j = mean|x_j|^alpha searched over alpha in
    [0, 1] for the least calibration output error after 4-bit quantization of
    W diag(s); its scaling identity X W^T = (X S^-1)(W S)^T moves magnitude
    from the activations to the weights without changing the layer).  The
    page fixes neither the grid nor the error measure's details; the reading:
    alpha = i / n_grid for i = 0 .. n_grid (both ends of [0, 1]; n_grid = 20
    as in the published method, Lin et al.); s = float32(max(mean_t |x_tj|^alpha,
    1e-4)) (the published method's floor, taken after the power; 0^0 = 1);
    the scaled weights float32(w * s) (one rounding of the exact product) are
    quantized by R2; the layer they give is X S^-1 (dequant)^T, so its error
    is ||X (W - W_hat)^T||_F^2 with W_hat = (q - zero) * scale / s in float64;
    the first alpha with the least error wins.  The activations' S^-1 is for
    the caller to fold into the producing operation.
R15 packed 4-bit zero points (linnet "Quantization": Int4GroupLinear's
    layout is ONNX Runtime's MatMulNBits, whose zero points are 4-bit values
    two a byte).  Per row, the zero points of groups 2j and 2j+1 share byte j,
    group 2j in the low nibble, as the codes are packed (R4); a row with an
    odd number of groups ends in a byte whose high nibble is padding, written
    as 0 and ignored when read.  The layer over packed zero points is the
    layer over the unpacked ones.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "QMAX_ASYM",
    "QMAX_SYM",
    "rint_half_even",
    "quantize_groups",
    "pack_uint4",
    "unpack_uint4",
    "dequantize_int4_groups",
    "linear_int4_groups",
    "bf16_round_bits",
    "bf16_bits_to_f64",
    "PREP_ROWS",
    "PREP_INPUTS",
    "prepared_bytes",
    "prepare_int4",
    "unprepare_int4",
    "QMIN_S4",
    "QMAX_S4",
    "quantize_int4_sym_f16",
    "pack_int4",
    "unpack_int4",
    "dequantize_int4_sym_f16",
    "linear_int4_sym_f16",
    "MX_BLOCK",
    "E2M1_VALUES",
    "quantize_mxfp4",
    "dequantize_mxfp4",
    "linear_mxfp4",
    "quantize_int4_rows",
    "dequantize_int4_rows",
    "linear_int4_rows",
    "gptq_quantize",
    "AWQ_FLOOR",
    "awq_scales",
    "awq_search",
    "awq_error",
    "pack_zero_points",
    "unpack_zero_points",
    "linear_int4_groups_zp4",
]

QMAX_ASYM = 15   # unsigned 4-bit codes 0..15 ("Per-Group INT4", 4.8 Quantization II)
QMAX_SYM = 7     # symmetric 4-bit limit Q = 2^(b-1) - 1 ("20. Quantization")


class OracleError(ValueError):
    """Input the pages' rules refuse (bad shapes, non-finite weights, codes > 15)."""


def rint_half_even(a):
    """Round to the nearest integer, halves to the even neighbour.

    tinyllm L8.5 section 2 ("Principles") fixes ties-to-even for every rounding;
    numpy's ``rint`` is IEEE round-to-nearest-even on float64.
    """
    return np.rint(np.asarray(a, dtype=np.float64))


def _check_groups(w: np.ndarray, group: int):
    if w.ndim != 2:
        raise OracleError("weight must be a matrix [Out, In]")
    if group < 1:
        raise OracleError("group must be positive")
    if w.shape[1] % group != 0:
        raise OracleError("group must divide In (the Int4GroupLinear layout has In/Group groups)")
    if not np.all(np.isfinite(w)):
        raise OracleError("weights must be finite")


def quantize_groups(w, group: int, symmetric: bool = False):
    """Round-to-nearest group quantizer.

    Args:
      w: float32 [N, K].  group: consecutive inputs per group (must divide K).
      symmetric: False -> asymmetric min/max scheme with a zero point (R2, R3);
                 True  -> symmetric absmax scheme stored offset by 8 (R4).
    Returns:
      q uint8 [N, K] in 0..15, scale float32 [N, K/group], zero uint8 [N, K/group].
    """
    w = np.asarray(w, dtype=np.float32)
    _check_groups(w, group)
    n, k = w.shape
    ng = k // group
    wg = w.reshape(n, ng, group).astype(np.float64)   # exact widening

    if symmetric:
        a = np.max(np.abs(wg), axis=-1)                     # group absmax (exact)
        nonzero = a > 0
        a_safe = np.where(nonzero, a, 1.0)
        scale = np.where(nonzero, (a_safe / QMAX_SYM), 1.0).astype(np.float32)
        c = rint_half_even((QMAX_SYM * wg) / a_safe[..., None])
        c = np.clip(c, -QMAX_SYM, QMAX_SYM)
        c = np.where(nonzero[..., None], c, 0.0)
        q = (c + 8).astype(np.uint8)
        zero = np.full((n, ng), 8, dtype=np.uint8)
        return q.reshape(n, k), scale, zero

    mn = np.min(wg, axis=-1)
    mx = np.max(wg, axis=-1)
    d = mx - mn                                          # float64 subtraction
    flat = d == 0
    d_safe = np.where(flat, 1.0, d)

    scale = np.where(flat, 1.0, d_safe / QMAX_ASYM).astype(np.float32)
    z_ratio = rint_half_even((-QMAX_ASYM * mn) / d_safe)
    z_flat = rint_half_even(-mn)
    zero = np.clip(np.where(flat, z_flat, z_ratio), 0, QMAX_ASYM)

    r_ratio = rint_half_even((QMAX_ASYM * wg) / d_safe[..., None])
    r_flat = rint_half_even(wg)
    r = np.where(flat[..., None], r_flat, r_ratio)
    q = np.clip(r + zero[..., None], 0, QMAX_ASYM)

    return (q.astype(np.uint8).reshape(n, k), scale, zero.astype(np.uint8))


def pack_uint4(q):
    """Two 4-bit codes per byte: element 2j in the low nibble, 2j+1 in the high nibble.

    The packing sentence of linnet "Quantization" and tinyllm L8.5 section 2
    ("Packing").  The last axis must have even length and every code must be
    at most 15; anything else is refused.
    """
    q = np.asarray(q)
    if q.shape[-1] % 2 != 0:
        raise OracleError("an odd number of codes cannot be packed two per byte")
    if q.size and (q.min() < 0 or q.max() > 15):
        raise OracleError("codes must lie in 0..15")
    q = q.astype(np.uint8)
    lo = q[..., 0::2]
    hi = q[..., 1::2]
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_uint4(packed):
    """Inverse of :func:`pack_uint4`: byte b -> (b & 0xF, b >> 4), unsigned."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0x0F)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def _codes_rows(packed, n: int, k: int):
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    return unpack_uint4(p)                             # [n, k]


def _dequant_exact(q_rows, scale_rows, zero_rows, group: int):
    """(q - zero) * scale per group as exact float64 values (R8)."""
    n, k = q_rows.shape
    ng = k // group
    qi = q_rows.reshape(n, ng, group).astype(np.float64)
    z = zero_rows.astype(np.float64)[..., None]
    s = scale_rows.astype(np.float32).astype(np.float64)[..., None]
    return ((qi - z) * s).reshape(n, k)


def bf16_round_bits(f32):
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Definition: keep the upper 16 bits of the float32 encoding after adding
    half of the dropped unit, with the tie going to an even kept value.
    Only finite inputs are expected here.
    """
    u = np.asarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dequantize_int4_groups(packed, scale, zero, n: int, k: int, group: int,
                           out: str = "f32"):
    """Group dequantization ``(q - zero) * scale`` (R7).

    packed uint8 [N, K/2] (or [N, K/G, G/2]); scale float32 [N, K/G];
    zero uint8 [N, K/G].  ``out="f32"`` returns float32 [N, K]; ``out="bf16"``
    returns the bfloat16 bit patterns (uint16 [N, K]) of the float32 result.
    """
    if group < 2 or group % 2 or k % group:
        raise OracleError("group must be even and divide K")
    q = _codes_rows(packed, n, k)
    w64 = _dequant_exact(q, np.asarray(scale).reshape(n, k // group),
                         np.asarray(zero).reshape(n, k // group), group)
    w32 = w64.astype(np.float32)                      # one rounding of an exact value
    if out == "f32":
        return w32
    if out == "bf16":
        return bf16_round_bits(w32)
    raise OracleError("out must be 'f32' or 'bf16'")


def linear_int4_groups(x, packed, scale, zero, n: int, k: int, group: int,
                       bias=None, order=None, rows=None, block_rows: int = 1024):
    """Exact-as-float64 value of ``y = x' . dequant(W)^T + bias`` (R6, R8).

    x: activations [M, K]; a uint16 array is read as bfloat16 bit patterns,
       anything else as real values.
    packed/scale/zero: the Int4GroupLinear tensors for W [N, K].
    bias: float32 [N] or None.  order: int32 [K] or None (gather, R6).
    rows: optional index array of output columns n to compute (the rest are
       not formed); the result then has shape [M, len(rows)].
    Returns float64 [M, N] (or [M, len(rows)]).
    """
    if group < 2 or group % 2 or k % group:
        raise OracleError("group must be even and divide K")
    x = np.asarray(x)
    xv = bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    if xv.ndim != 2 or xv.shape[1] != k:
        raise OracleError("x must be [M, K]")
    if order is not None:
        order = np.asarray(order, dtype=np.int64)
        if order.shape != (k,) or (k and (order.min() < 0 or order.max() >= k)):
            raise OracleError("order must hold K indices in [0, K)")
        xv = xv[:, order]                               # gather: x'[m,k] = x[m, order[k]]
    ng = k // group
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    s = np.asarray(scale, dtype=np.float32).reshape(n, ng)
    z = np.asarray(zero, dtype=np.uint8).reshape(n, ng)
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.empty((xv.shape[0], idx.size), dtype=np.float64)
    for b0 in range(0, idx.size, block_rows):
        sel = idx[b0:b0 + block_rows]
        w_rows = _dequant_exact(unpack_uint4(p[sel]), s[sel], z[sel], group)
        y[:, b0:b0 + sel.size] = xv @ w_rows.T
    if bias is not None:
        y += np.asarray(bias, dtype=np.float32).astype(np.float64)[idx][None, :]
    return y


# ---------------------------------------------------------------------------
# Prepared (fragment-ordered) weights, R9
# ---------------------------------------------------------------------------

PREP_ROWS = 16      # outputs per block
PREP_INPUTS = 128   # inputs per block (64 packed bytes of each row)


def prepared_bytes(n: int, k: int) -> int:
    """Size of the prepared layout of an [n, k] weight: whole 16 x 128 blocks."""
    return -(-n // PREP_ROWS) * -(-k // PREP_INPUTS) * PREP_ROWS * PREP_INPUTS // 2


def _prep_dims(n: int, k: int):
    if n < 0 or k < 0 or k % 32:
        raise OracleError("prepared weights need k a multiple of 32")
    return -(-n // PREP_ROWS), -(-k // PREP_INPUTS)


def prepare_int4(packed, n: int, k: int):
    """Canonical packed rows [n, k/2] -> prepared blocks (R9), a flat uint8 array.

    Blocks are ordered (tile t, step s); block (t, s) is the 4 x 16 x 16-byte
    array [q][c][byte] = packed row 16t + c, bytes 64 s + 16 q + byte.
    """
    nt, ns = _prep_dims(n, k)
    rows = np.zeros((nt * PREP_ROWS, ns * PREP_INPUTS // 2), dtype=np.uint8)
    rows[:n, :k // 2] = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    # [t][c][s][q][byte] -> [t][s][q][c][byte]
    blocks = rows.reshape(nt, PREP_ROWS, ns, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(blocks).reshape(-1)


def unprepare_int4(prepared, n: int, k: int):
    """Inverse of :func:`prepare_int4`: prepared blocks -> packed rows [n, k/2]."""
    nt, ns = _prep_dims(n, k)
    blocks = np.asarray(prepared, dtype=np.uint8).reshape(nt, ns, 4, PREP_ROWS, 16)
    rows = blocks.transpose(0, 3, 1, 2, 4).reshape(nt * PREP_ROWS, ns * PREP_INPUTS // 2)
    return np.ascontiguousarray(rows[:n, :k // 2])


# ---------------------------------------------------------------------------
# Signed int4 groups with float16 scales, R10
# ---------------------------------------------------------------------------

QMIN_S4 = -8   # 4-bit two's complement range (tinyllm L8.5, "int4 per group")
QMAX_S4 = 7


def quantize_int4_sym_f16(w, group: int = 32):
    """Symmetric signed int4 per group with a float16 scale (R10).

    tinyllm L8.5 section 2, "int4 per group": s16 = float16(amax / 7), codes
    rint(w / s16) against the stored float16 scale; zero or underflowing
    groups get codes 0; a float16 overflow is an error.
    Args: w float32 [N, K]; group divides K and is even.
    Returns: codes int8 [N, K] in -8..7, scale float16 [N, K/group].
    """
    w = np.asarray(w, dtype=np.float32)
    _check_groups(w, group)
    if group % 2:
        raise OracleError("an odd group cannot be packed two per byte")
    n, k = w.shape
    ng = k // group
    wg = w.reshape(n, ng, group)
    amax = np.max(np.abs(wg), axis=-1)                       # float32, exact
    q32 = amax / np.float32(QMAX_S4)                         # float32 quotient
    with np.errstate(over="ignore"):
        s16 = q32.astype(np.float16)                         # round to float16, ties to even
    if not np.all(np.isfinite(s16)):
        raise OracleError("a group scale overflows float16")
    s = s16.astype(np.float32)                               # the stored value, exactly
    live = s > 0
    quot = wg / np.where(live, s, np.float32(1))[..., None]  # float32 quotient against s16
    c = np.clip(rint_half_even(quot), QMIN_S4, QMAX_S4)
    c = np.where(live[..., None], c, 0.0)
    return c.astype(np.int8).reshape(n, k), s16


def pack_int4(c):
    """Two signed 4-bit codes per byte, two's complement, even element low.

    tinyllm L8.5 section 2, "Packing": nibble = c & 0xF.  Codes outside
    -8..7 and odd widths are refused.
    """
    c = np.asarray(c)
    if c.shape[-1] % 2 != 0:
        raise OracleError("an odd number of codes cannot be packed two per byte")
    if c.size and (c.min() < QMIN_S4 or c.max() > QMAX_S4):
        raise OracleError("signed 4-bit codes lie in -8..7")
    nib = (c.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_int4(packed):
    """Inverse of :func:`pack_int4`: each nibble sign-extended (v >= 8 is v - 16)."""
    p = np.asarray(packed, dtype=np.uint8)
    nib = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int16)
    nib[..., 0::2] = p & np.uint8(0x0F)
    nib[..., 1::2] = p >> np.uint8(4)
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


def _sym_exact(c_rows, s16_rows, group: int):
    """c * s16 per group as exact float64 values (R10)."""
    n, k = c_rows.shape
    s = np.asarray(s16_rows, dtype=np.float16).astype(np.float64)[..., None]
    return (c_rows.reshape(n, k // group, group).astype(np.float64) * s).reshape(n, k)


def dequantize_int4_sym_f16(packed, scale16, n: int, k: int, group: int, out: str = "f32"):
    """``c * s16`` per group (R10); float32 [N, K], or bfloat16 bit patterns of it."""
    if group < 2 or group % 2 or k % group:
        raise OracleError("group must be even and divide K")
    c = unpack_int4(np.asarray(packed, dtype=np.uint8).reshape(n, k // 2))
    w32 = _sym_exact(c, np.asarray(scale16).reshape(n, k // group), group).astype(np.float32)
    if out == "f32":
        return w32
    if out == "bf16":
        return bf16_round_bits(w32)
    raise OracleError("out must be 'f32' or 'bf16'")


def linear_int4_sym_f16(x, packed, scale16, n: int, k: int, group: int,
                        bias=None, order=None, rows=None, block_rows: int = 1024):
    """Exact-as-float64 value of ``y = x' . dequant(W)^T + bias`` for R10 weights.

    Arguments as :func:`linear_int4_groups`, with float16 scales and no zero.
    """
    if group < 2 or group % 2 or k % group:
        raise OracleError("group must be even and divide K")
    x = np.asarray(x)
    xv = bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    if xv.ndim != 2 or xv.shape[1] != k:
        raise OracleError("x must be [M, K]")
    if order is not None:
        order = np.asarray(order, dtype=np.int64)
        if order.shape != (k,) or (k and (order.min() < 0 or order.max() >= k)):
            raise OracleError("order must hold K indices in [0, K)")
        xv = xv[:, order]
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    s = np.asarray(scale16, dtype=np.float16).reshape(n, k // group)
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.empty((xv.shape[0], idx.size), dtype=np.float64)
    for b0 in range(0, idx.size, block_rows):
        sel = idx[b0:b0 + block_rows]
        y[:, b0:b0 + sel.size] = xv @ _sym_exact(unpack_int4(p[sel]), s[sel], group).T
    if bias is not None:
        y += np.asarray(bias, dtype=np.float32).astype(np.float64)[idx][None, :]
    return y


# ---------------------------------------------------------------------------
# MXFP4: E2M1 codes in blocks of 32 with an E8M0 scale, R11
# ---------------------------------------------------------------------------

MX_BLOCK = 32
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)   # magnitudes of codes 0..7 (tinyllm "MXFP4")


def _e2m1_round(v):
    """Nearest E2M1 code of real values v (float64): ties to the even code, saturating at 6."""
    mags = np.asarray(E2M1_VALUES)
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - mags)                            # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                           # one or two nearest codes
    even = cand & ((np.arange(8) % 2) == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (idx + np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def _e8m0_value(e):
    """X = 2^(e - 127) as float64 (255, not a number in E8M0, gives NaN)."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).astype(np.int64)))


def _e2m1_value(c):
    c = np.asarray(c, dtype=np.uint8)
    v = np.asarray(E2M1_VALUES)[c & 7]
    return np.where(c & 8, -v, v)


def quantize_mxfp4(w):
    """MXFP4 quantizer (R11).  w float32 [N, K], K a multiple of 32.

    Returns codes uint8 [N, K] (0..15, E2M1 bit patterns) and scales uint8
    [N, K/32] (E8M0).  Non-finite weights are refused.
    """
    w = np.asarray(w, dtype=np.float32)
    _check_groups(w, MX_BLOCK)
    n, k = w.shape
    wb = w.reshape(n, k // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.max(np.abs(wb), axis=-1)
    _, ex = np.frexp(amax)                                   # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, np.clip(ex - 1 - 2 + 127, 0, 254), 0).astype(np.int64)
    x_scale = _e8m0_value(e)
    codes = _e2m1_round(wb / x_scale[..., None])              # exact: X is a power of two
    return codes.reshape(n, k), e.astype(np.uint8)


def dequantize_mxfp4(blocks, scales, n: int, k: int, out: str = "f32"):
    """E2M1 value * 2^(e - 127) per block of 32 (R11); float32 [N, K] or bf16 bits."""
    if k % MX_BLOCK:
        raise OracleError("K must be a multiple of 32")
    c = unpack_uint4(np.asarray(blocks, dtype=np.uint8).reshape(n, k // 2))
    x_scale = np.repeat(_e8m0_value(np.asarray(scales).reshape(n, k // MX_BLOCK)), MX_BLOCK, axis=1)
    w32 = (_e2m1_value(c) * x_scale).astype(np.float32)
    if out == "f32":
        return w32
    if out == "bf16":
        return bf16_round_bits(w32)
    raise OracleError("out must be 'f32' or 'bf16'")


def linear_mxfp4(x, blocks, scales, n: int, k: int, bias=None, rows=None, block_rows: int = 1024):
    """Exact-as-float64 value of ``y = x . dequant(W)^T + bias`` for MXFP4 weights (R11)."""
    if k % MX_BLOCK:
        raise OracleError("K must be a multiple of 32")
    x = np.asarray(x)
    xv = bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    if xv.ndim != 2 or xv.shape[1] != k:
        raise OracleError("x must be [M, K]")
    p = np.asarray(blocks, dtype=np.uint8).reshape(n, k // 2)
    e = np.asarray(scales, dtype=np.uint8).reshape(n, k // MX_BLOCK)
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.empty((xv.shape[0], idx.size), dtype=np.float64)
    for b0 in range(0, idx.size, block_rows):
        sel = idx[b0:b0 + block_rows]
        w = _e2m1_value(unpack_uint4(p[sel])) * np.repeat(_e8m0_value(e[sel]), MX_BLOCK, axis=1)
        y[:, b0:b0 + sel.size] = xv @ w.T
    if bias is not None:
        y += np.asarray(bias, dtype=np.float32).astype(np.float64)[idx][None, :]
    return y


# ---------------------------------------------------------------------------
# Int4Linear: signed int4 codes with one float32 scale a row, R12
# ---------------------------------------------------------------------------

def quantize_int4_rows(w):
    """Symmetric signed int4 per row (R12).  w float32 [N, K], K even.

    Returns codes int8 [N, K] in -8..7 and scale float32 [N].
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise OracleError("weight must be a matrix [Out, In]")
    if w.shape[1] % 2:
        raise OracleError("an odd number of inputs cannot be packed two per byte")
    if not np.all(np.isfinite(w)):
        raise OracleError("weights must be finite")
    amax = np.max(np.abs(w), axis=1) if w.shape[1] else np.zeros(w.shape[0], np.float32)
    s = (amax / np.float32(QMAX_S4)).astype(np.float32)          # float32 quotient
    live = s > 0
    quot = w / np.where(live, s, np.float32(1))[:, None]          # float32 quotient
    c = np.clip(rint_half_even(quot), QMIN_S4, QMAX_S4)
    c = np.where(live[:, None], c, 0.0)
    return c.astype(np.int8), s


def _rows_exact(c_rows, s_rows):
    return c_rows.astype(np.float64) * np.asarray(s_rows, dtype=np.float32).astype(np.float64)[:, None]


def dequantize_int4_rows(packed, scale, n: int, k: int, out: str = "f32"):
    """``c * s`` per row, rounded once to float32 (R12); float32 [N, K] or bf16 bits."""
    c = unpack_int4(np.asarray(packed, dtype=np.uint8).reshape(n, k // 2))
    w32 = _rows_exact(c, np.asarray(scale).reshape(n)).astype(np.float32)
    if out == "f32":
        return w32
    if out == "bf16":
        return bf16_round_bits(w32)
    raise OracleError("out must be 'f32' or 'bf16'")


def linear_int4_rows(x, packed, scale, n: int, k: int, bias=None, order=None, rows=None,
                     block_rows: int = 1024):
    """Exact-as-float64 value of ``y = x' . dequant(W)^T + bias`` for Int4Linear weights (R12)."""
    x = np.asarray(x)
    xv = bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    if xv.ndim != 2 or xv.shape[1] != k:
        raise OracleError("x must be [M, K]")
    if order is not None:
        order = np.asarray(order, dtype=np.int64)
        if order.shape != (k,) or (k and (order.min() < 0 or order.max() >= k)):
            raise OracleError("order must hold K indices in [0, K)")
        xv = xv[:, order]
    p = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2)
    s = np.asarray(scale, dtype=np.float32).reshape(n)
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.empty((xv.shape[0], idx.size), dtype=np.float64)
    for b0 in range(0, idx.size, block_rows):
        sel = idx[b0:b0 + block_rows]
        y[:, b0:b0 + sel.size] = xv @ _rows_exact(unpack_int4(p[sel]), s[sel]).T
    if bias is not None:
        y += np.asarray(bias, dtype=np.float32).astype(np.float64)[idx][None, :]
    return y


# ---------------------------------------------------------------------------
# GPTQ, R13
# ---------------------------------------------------------------------------

def _asym_group_params(wg):
    """R2/R3 scale and zero of each row of a group block wg [N, G] (float64 values)."""
    mn, mx = wg.min(axis=1), wg.max(axis=1)
    d = mx - mn
    flat = d == 0
    d_safe = np.where(flat, 1.0, d)
    scale = np.where(flat, 1.0, d_safe / QMAX_ASYM).astype(np.float32)
    zero = np.clip(np.where(flat, rint_half_even(-mn), rint_half_even((-QMAX_ASYM * mn) / d_safe)), 0, QMAX_ASYM)
    return scale, zero, flat, d_safe


def gptq_quantize(w, x, group: int, act_order: bool = False, damp: float = 0.01):
    """GPTQ of one layer (R13), in float64.

    w: float32 [N, K]; x: calibration activations [T, K] (a uint16 array is
    read as bfloat16 bit patterns).  Returns (q uint8 [N, K], scale float32
    [N, K/G], zero uint8 [N, K/G], order int32 [K] or None), the columns of q
    (and the groups) in visiting order; the layer gathers its inputs through
    `order` (R6).
    """
    w = np.asarray(w, dtype=np.float32)
    _check_groups(w, group)
    n, k = w.shape
    x = np.asarray(x)
    xv = bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    if xv.ndim != 2 or xv.shape[1] != k:
        raise OracleError("calibration inputs must be [T, K]")
    W = w.astype(np.float64)
    H = xv.T @ xv
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    W[:, dead] = 0.0
    perm = None
    if act_order:
        perm = np.argsort(-np.diag(H), kind="stable")
        W = W[:, perm]
        H = H[perm][:, perm]
    H = H + damp * np.mean(np.diag(H)) * np.eye(k)
    U = np.linalg.cholesky(np.linalg.inv(H)).T                 # upper, H^-1 = U^T U
    q = np.zeros((n, k), dtype=np.uint8)
    ng = k // group
    scale = np.zeros((n, ng), dtype=np.float32)
    zero = np.zeros((n, ng), dtype=np.uint8)
    for i in range(k):
        g = i // group
        if i % group == 0:
            sc, zr, flat, d_safe = _asym_group_params(W[:, i:i + group])
            scale[:, g], zero[:, g] = sc, zr
        col = W[:, i]
        r = np.where(flat, rint_half_even(col), rint_half_even((QMAX_ASYM * col) / d_safe))
        qi = np.clip(r + zero[:, g], 0, QMAX_ASYM)
        q[:, i] = qi
        deq = (qi - zero[:, g].astype(np.float64)) * scale[:, g].astype(np.float64)
        err = (col - deq) / U[i, i]
        W[:, i + 1:] -= np.outer(err, U[i, i + 1:])
    return q, scale, zero, (None if perm is None else perm.astype(np.int32))



AWQ_FLOOR = 1e-4


def awq_scales(mean_abs, alpha: float):
    """R14 per-channel scales: float32(max(mean_abs^alpha, 1e-4))."""
    return np.maximum(np.power(np.asarray(mean_abs, np.float64), float(alpha)), AWQ_FLOOR).astype(np.float32)


def awq_search(w, x, group: int, n_grid: int = 20):
    """AWQ scale search for one layer (R14), in float64.

    w: float32 [N, K]; x: calibration activations [T, K], T >= 1 (a uint16
    array is read as bfloat16 bit patterns).  Returns (q uint8 [N, K], scale
    float32 [N, K/G], zero uint8 [N, K/G]) of the scaled weights W diag(s),
    s float32 [K], the chosen grid index, and the error of every grid point
    (float64 [n_grid + 1]).
    """
    w = np.asarray(w, dtype=np.float32)
    _check_groups(w, group)
    n, k = w.shape
    if n_grid < 1:
        raise OracleError("n_grid must be positive")
    x = np.asarray(x)
    xv = bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    if xv.ndim != 2 or xv.shape[1] != k or xv.shape[0] < 1:
        raise OracleError("calibration inputs must be [T, K] with T >= 1")
    mean_abs = np.abs(xv).mean(axis=0)
    losses = np.zeros(n_grid + 1)
    best = None
    for i in range(n_grid + 1):
        s = awq_scales(mean_abs, i / n_grid)
        losses[i], q, sc, zr = awq_error(w, xv, group, s)
        if best is None or losses[i] < losses[best[0]]:
            best = (i, q, sc, zr, s)
    i, q, sc, zr, s = best
    return q, sc, zr, s, i, losses


def awq_error(w, xv, group: int, s):
    """R14 error of one scale vector: quantize float32(w * s) by R2 and return
    (||X (W - W_hat)^T||_F^2, q, scale, zero), W_hat = (q - zero) * scale / s in
    float64; xv float64 [T, K]."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    w64 = w.astype(np.float64)
    s64 = np.asarray(s, np.float32).astype(np.float64)
    ws = (w64 * s64).astype(np.float32)
    q, sc, zr = quantize_groups(ws, group)
    deq = (q.reshape(n, k // group, group).astype(np.float64) - zr[:, :, None]) * sc[:, :, None]
    w_hat = deq.reshape(n, k) / s64
    e = np.asarray(xv, np.float64) @ (w64 - w_hat).T
    return float(np.sum(e * e)), q, sc, zr


def pack_zero_points(zero):
    """R15: zero points [N, G_n] (0..15) -> bytes [N, ceil(G_n / 2)], group 2j low."""
    z = np.asarray(zero)
    if z.ndim != 2:
        raise OracleError("zero points must be [N, groups]")
    if z.size and (z.min() < 0 or z.max() > 15):
        raise OracleError("zero points must lie in 0..15")
    z = z.astype(np.uint8)
    if z.shape[1] % 2:
        z = np.concatenate([z, np.zeros((z.shape[0], 1), np.uint8)], axis=1)   # the padding nibble
    return pack_uint4(z)


def unpack_zero_points(packed, n: int, ngroups: int):
    """Inverse of :func:`pack_zero_points`: [N, ceil(G_n / 2)] bytes -> [N, G_n]."""
    p = np.asarray(packed, dtype=np.uint8).reshape(n, (ngroups + 1) // 2)
    return unpack_uint4(p)[:, :ngroups]


def linear_int4_groups_zp4(x, packed, scale, zero_packed, n: int, k: int, group: int,
                           bias=None, order=None, rows=None):
    """The linear layer (R6, R8) over packed zero points (R15)."""
    if group < 1 or k % group:
        raise OracleError("group must divide K")
    zero = unpack_zero_points(zero_packed, n, k // group)
    return linear_int4_groups(x, packed, scale, zero, n, k, group, bias=bias, order=order, rows=rows)
