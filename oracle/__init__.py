"""CPU oracle for the group-wise 4-bit weight-only linear layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library never imports, links or calls anything here, and
nothing here calls the HIP library.  See ``woq_ref`` for the definitions and
the readings of the pages they follow.
"""
from .woq_ref import (  # noqa: F401
    E2M1_VALUES,
    MX_BLOCK,
    QMAX_ASYM,
    QMAX_S4,
    QMAX_SYM,
    QMIN_S4,
    OracleError,
    PREP_INPUTS,
    PREP_ROWS,
    bf16_bits_to_f64,
    bf16_round_bits,
    dequantize_int4_groups,
    dequantize_int4_rows,
    dequantize_int4_sym_f16,
    dequantize_mxfp4,
    AWQ_FLOOR,
    awq_scales,
    awq_error,
    awq_search,
    gptq_quantize,
    linear_int4_groups,
    linear_int4_groups_zp4,
    linear_int4_rows,
    linear_int4_sym_f16,
    linear_mxfp4,
    pack_int4,
    pack_zero_points,
    pack_uint4,
    prepare_int4,
    quantize_int4_sym_f16,
    quantize_mxfp4,
    prepared_bytes,
    quantize_groups,
    quantize_int4_rows,
    rint_half_even,
    unpack_int4,
    unpack_zero_points,
    unpack_uint4,
    unprepare_int4,
)
