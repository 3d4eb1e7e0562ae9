"""The C-ABI library on a host without a GPU: it loads, exports every symbol
include/woq.h declares, and its pure-host functions and argument checks
behave as documented.  Only calls that return before any HIP call are made.
"""
import ctypes
import re
from pathlib import Path

import pytest

import weight_only_quantization_amd as woq

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "woq.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(woq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return woq.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("woq_quantize_groups", "woq_pack_uint4", "woq_unpack_uint4",
                 "woq_dequantize_int4_groups", "woq_linear_int4_groups",
                 "woq_linear_workspace_bytes", "woq_linear_plan", "woq_status_str"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libwoq.so does not export {name}"


def test_status_strings(lib):
    for code in range(10):
        s = lib.woq_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.woq_status_str(99).decode() == "unknown status"
    assert lib.woq_version() >= 100


@pytest.mark.parametrize("m,n,k,g,path", [
    (1, 4096, 4096, 128, "rows_dot2"), (4, 14336, 4096, 32, "rows_dot2"),
    (1, 8192, 28672, 128, "rows_dot2"), (1, 64, 40960, 128, "skinny_mfma"),
    (2, 4096, 32768, 64, "rows_dot2"), (1, 4096, 32800, 32, "skinny_mfma"),
    (5, 4096, 4096, 128, "skinny_mfma"), (16, 14336, 4096, 32, "skinny_mfma"),
    (17, 4096, 4096, 128, "smallm_lds"), (32, 14336, 4096, 256, "skinny_mfma"),
    (33, 4096, 4096, 128, "smallm_lds"), (64, 14336, 4096, 32, "skinny_mfma"),
    (7, 4096, 14336, 128, "skinny_mfma"), (8, 4096, 14336, 128, "smallm_lds"),
    (15, 4096, 4096, 128, "skinny_mfma"), (16, 4096, 14336, 128, "smallm_lds"),
    (64, 4096, 14336, 256, "smallm_lds"), (64, 4096, 14336, 32, "skinny_mfma"),
    (48, 1024, 4096, 128, "smallm_lds"), (16, 12800, 4096, 128, "skinny_mfma"),
    (8, 1024, 4096, 128, "smallm_lds"), (8, 4096, 4096, 128, "skinny_mfma"), (7, 1024, 4096, 128, "skinny_mfma"),
    (8, 1024, 4096, 32, "skinny_mfma"), (12, 4096, 14336, 256, "smallm_lds"), (12, 4096, 14336, 64, "skinny_mfma"),
    (65, 4096, 4096, 128, "gemm_mfma"), (128, 14336, 4096, 32, "skinny_mfma"),
    (128, 4096, 14336, 128, "gemm_mfma"), (129, 14336, 4096, 128, "gemm_mfma"), (2048, 14336, 4096, 128, "gemm_mfma"),
    (0, 64, 256, 32, "none"), (3, 64, 0, 32, "bias_fill"),
])
def test_plan_paths(m, n, k, g, path):
    assert f"path={path}" in woq.linear_plan(m, n, k, g)


def test_plan_smallm_lds(monkeypatch):
    # 16..64 rows on layers under 800 tiles of 16 rows: 8-step K ranges from K = 8192
    # (two tiles a wave above 32 rows), else 4; the partial buffer is workspace
    for (m, n, k, g), (t, s, r) in (((16, 4096, 14336, 128), (1, 8, 14)), ((64, 4096, 14336, 128), (2, 8, 14)),
                                    ((32, 4096, 14336, 32), (1, 8, 14)), ((24, 4096, 4096, 128), (1, 4, 8)),
                                    ((64, 1024, 4160, 64), (1, 4, 9))):
        plan = woq.linear_plan(m, n, k, g)
        assert f"path=smallm_lds act_tiles={1 if m <= 16 else (2 if m <= 32 else 4)} " in plan, plan
        assert f"weight_tiles_per_wave={t} waves=8 steps_per_range={s} k_ranges={r} " in plan, plan
        part = r * m * n * 4
        assert woq.linear_workspace_bytes(m, n, k, g, False) == (part + 255) // 256 * 256
        xg = (m * k * 2 + 255) // 256 * 256
        assert woq.linear_workspace_bytes(m, n, k, g, True) == xg + (part + 255) // 256 * 256
    # tuning aids: "0" keeps calls off the path, "T,S" forces a shape from 5 rows up
    monkeypatch.setenv("WOQ_SM", "0")
    assert "path=skinny_mfma" in woq.linear_plan(16, 4096, 14336, 128)
    monkeypatch.setenv("WOQ_SM", "2,4")
    plan = woq.linear_plan(5, 14336, 4096, 128)
    assert "path=smallm_lds" in plan and "weight_tiles_per_wave=2 waves=8 steps_per_range=4 k_ranges=8" in plan
    monkeypatch.setenv("WOQ_SM", "2,8")   # two tiles of 8-step ranges at 64 rows and group 32: LDS too small
    assert "path=smallm_lds" not in woq.linear_plan(64, 4096, 14336, 32)


def test_plan_decode_kernels(monkeypatch):
    # canonical rows at m <= 4 stream through the row kernel: rows per workgroup by shape
    for (m, n, k, g), u in (((1, 14336, 4096, 128), 4), ((1, 4096, 14336, 128), 16), ((1, 4096, 4096, 128), 4),
                            ((1, 1024, 4096, 128), 4), ((3, 4096, 4096, 128), 4), ((2, 28672, 4096, 128), 4),
                            ((4, 14336, 4096, 64), 4)):
        plan = woq.linear_plan(m, n, k, g)
        assert f"path=rows_dot2 rows_per_group={u} waves={(k + 2047) // 2048} " in plan, plan
    # 3 and 4 rows of layers with >= 2^25 weights and groups >= 128 take the small-M MFMA kernel,
    # or the tile GEMV when K >= 8192
    for m, n, k, g in ((3, 14336, 4096, 128), (4, 8192, 4096, 128)):
        assert "path=skinny_mfma" in woq.linear_plan(m, n, k, g)
    for m, n, k, g in ((4, 4096, 14336, 256), (3, 4096, 14336, 128), (2, 4096, 14336, 128), (2, 8192, 28672, 128)):
        assert "path=gemv_mfma" in woq.linear_plan(m, n, k, g)
    for m, n, k, g in ((2, 14336, 4096, 128), (2, 4096, 14336, 64), (1, 4096, 14336, 128)):
        assert "path=rows_dot2" in woq.linear_plan(m, n, k, g)
    # (where the tile GEMV's staging does not fit in LDS, the small-M kernel keeps them)
    assert "path=skinny_mfma" in woq.linear_plan(4, 8192, 28672, 128)
    monkeypatch.setenv("WOQ_DECODE_MFMA", "1")
    assert "path=gemv_mfma" in woq.linear_plan(1, 4096, 4096, 128)
    assert "path=gemv_mfma" in woq.linear_plan(4, 14336, 4096, 128)


@pytest.mark.parametrize("m,n,tail", [
    (2048, 14336, 2048),    # 896 tiles: the 128 of the last round become 256 tiles of 64 rows
    (2048, 4096, 0),        # 256 tiles: one full round
    (1024, 14336, 0),       # 448 tiles: the last round is 3/4 full
    (200, 33064, 296),      # ragged rows and columns: 2 trailing tile columns
    (384, 16384, 0),        # 192 tiles: three quarters of the chip, one round
])
def test_plan_tail_split(m, n, tail):
    plan = woq.linear_plan(m, n, 256, 128)
    fields = dict(f.split("=", 1) for f in plan.split())
    assert fields["path"] == "gemm_mfma" and fields["tile"] == "128x256"
    assert int(fields["tail_cols"]) == tail
    tm, tn = -(-m // 128), -(-n // 256)
    cols = -(-tail // 256)
    assert int(fields["grid"]) == tm * (tn - cols) + (-(-m // 64)) * cols


@pytest.mark.parametrize("m,n,k,group,tile,splits", [
    (256, 1024, 4096, 128, "128x64", 8),     # 8 tiles of 128 x 256 x 8 ranges: a quarter of the chip
    (256, 4096, 4096, 128, "128x256", 8),    # 32 tiles, 32 steps: 8 ranges of 4
    (256, 4096, 14336, 128, "128x256", 8),
    (256, 14336, 4096, 128, "128x256", 2),   # 112 tiles
    (512, 1024, 4096, 128, "128x64", 4),     # 128 x 256 would fill exactly half the chip
    (512, 14336, 4096, 128, "128x256", 1),   # 224 tiles
    (128, 4096, 14336, 128, "128x256", 14),  # above 64 rows the small-M kernel wants >= 4 tiles of 16 rows a workgroup
    (96, 1024, 4096, 128, "128x64", 8),      # at most 16 ranges of >= 4 steps
    (300, 1000, 4160, 64, "128x64", 5),      # 33 steps: ranges of 8, the last holds one
    (129, 256, 256, 128, "128x64", 1),       # 2 steps: too short to split
    (384, 16384, 4096, 128, "128x256", 1),   # 192 tiles of 128 x 256
    (2048, 4096, 14336, 128, "128x256", 1),
])
def test_plan_split_k(m, n, k, group, tile, splits):
    """Above 64 rows: tiles of 128 x 256 unless, even split over K, they would
    fill at most half the chip (then 128 x 64); a grid under three quarters of
    the chip takes K ranges (each an even number of at least 4 steps, at most
    16 ranges) until it fills one round."""
    fields = dict(f.split("=", 1) for f in woq.linear_plan(m, n, k, group).split())
    assert fields["path"] == "gemm_mfma" and fields["tile"] == tile
    assert int(fields["k_splits"]) == splits
    bm, bn = map(int, tile.split("x"))
    tiles = -(-m // bm) * -(-n // bn)
    assert int(fields["grid"]) == tiles * splits
    nsteps = -(-k // 128)
    if splits > 1:
        assert tiles * splits <= 256 and splits <= 16
        sps = -(-nsteps // splits)
        sps += sps & 1
        assert -(-nsteps // sps) == splits and sps >= 4
        # the partial outputs, float32 [splits][m][n], are part of the workspace
        one = woq.linear_workspace_bytes(m, n, k, group, False)
        assert one >= splits * m * n * 4
    else:
        assert tiles >= 192 or nsteps < 8 or (tiles > 128 and 256 // tiles < 2)


def test_plan_mentions_gather_for_act_order():
    assert "gather" in woq.linear_plan(1, 8192, 28672, 128, has_order=True)


def test_workspace_sizes():
    assert woq.linear_workspace_bytes(1, 4096, 4096, 128, False) == 0
    ws = woq.linear_workspace_bytes(1, 8192, 28672, 128, True)
    assert ws >= 1 * 28672 * 2 and ws % 256 == 0
    big = woq.linear_workspace_bytes(2048, 14336, 4096, 128, False)
    assert big >= 2048 * 4096 * 2 + (4096 // 128) * 2048 * 4


@pytest.mark.parametrize("m,n,k,g,status", [
    (-1, 64, 256, 32, "WOQ_EINVAL"),
    (1, 64, 256, 48, "WOQ_EGROUP"),      # 48 does not divide 256
    (1, 64, 240, 48, "WOQ_EUNSUPPORTED"),  # valid layout, no kernel for group 48
    (1, 64, 256, 33, "WOQ_EGROUP"),      # odd group
    (1, 64, 256, 0, "WOQ_EGROUP"),
    (1, 64, 96, 64, "WOQ_EGROUP"),       # 64 does not divide 96
    (1, 1 << 31, 256, 32, "WOQ_EUNSUPPORTED"),
])
def test_linear_rejects_bad_shapes_before_any_launch(lib, m, n, k, g, status):
    rc = lib.woq_linear_int4_groups(None, m, None, None, None, None, None, n, k, g, 1,
                                    None, None, 0, None)
    assert woq.STATUS[rc] == status


def test_linear_rejects_null_pointers_and_bad_dtype(lib):
    fake = ctypes.c_void_p(4096)   # never dereferenced: validation fails first
    rc = lib.woq_linear_int4_groups(None, 1, fake, fake, fake, None, None, 64, 256, 32, 1,
                                    fake, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EINVAL"
    rc = lib.woq_linear_int4_groups(fake, 1, fake, fake, fake, None, None, 64, 256, 32, 7,
                                    fake, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EINVAL"
    rc = lib.woq_linear_int4_groups(fake, 1, fake, fake, fake, None, None, 64, 256, 32, 1,
                                    None, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EINVAL"


def test_linear_rejects_misalignment_and_missing_workspace(lib):
    a16 = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    rc = lib.woq_linear_int4_groups(odd, 1, a16, a16, a16, None, None, 64, 256, 32, 1,
                                    a16, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EALIGN"
    rc = lib.woq_linear_int4_groups(a16, 1, odd, a16, a16, None, None, 64, 256, 32, 1,
                                    a16, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EALIGN"
    # act-order needs a gather buffer
    rc = lib.woq_linear_int4_groups(a16, 1, a16, a16, a16, None, a16, 64, 256, 32, 1,
                                    a16, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EWORKSPACE"
    # the GEMM path needs its pre-pass buffers
    rc = lib.woq_linear_int4_groups(a16, 200, a16, a16, a16, None, None, 64, 256, 32, 1,
                                    a16, a16, 16, None)
    assert woq.STATUS[rc] == "WOQ_EWORKSPACE"


def test_grouped_call_checks_every_matrix_first(lib):
    a16 = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    P = lambda *v: (ctypes.c_void_p * len(v))(*v)
    N = lambda *v: (ctypes.c_int64 * len(v))(*v)
    ok3 = P(a16, a16, a16)

    def call(count, packed=ok3, scale=ok3, zero=ok3, bias=None, n=N(64, 32, 16), k=256, g=32,
             prepared=0, ydt=1, y=ok3, m=1):
        return woq.STATUS[lib.woq_linear_int4_groups_grouped(a16, m, count, packed, scale, zero, bias, n, k,
                                                             g, prepared, ydt, y, None, 0, None)]

    assert call(0) == "WOQ_EINVAL" and call(5) == "WOQ_EINVAL"
    assert call(3, packed=None) == "WOQ_EINVAL" and call(3, n=None) == "WOQ_EINVAL"
    assert call(3, prepared=2) == "WOQ_EINVAL" and call(3, ydt=7) == "WOQ_EINVAL"
    assert call(3, y=P(a16, None, a16)) == "WOQ_EINVAL"            # one output missing
    assert call(3, zero=P(a16, a16, odd)) == "WOQ_EALIGN"         # checked for the last matrix too
    assert call(3, n=N(64, -1, 16)) == "WOQ_EINVAL"
    assert call(2, g=48) == "WOQ_EGROUP"
    assert call(3, m=0) == "WOQ_OK"                                # nothing to do
    assert call(2, n=N(0, 0)) == "WOQ_OK"


def test_empty_calls_are_noops(lib):
    assert lib.woq_linear_int4_groups(None, 0, None, None, None, None, None, 64, 256, 32, 1,
                                      None, None, 0, None) == 0
    assert lib.woq_linear_int4_groups(None, 4, None, None, None, None, None, 0, 256, 32, 1,
                                      None, None, 0, None) == 0
    assert lib.woq_quantize_groups(None, 0, 256, 32, 0, None, None, None, None) == 0
    assert lib.woq_pack_uint4(None, 0, None, None) == 0
    assert lib.woq_unpack_uint4(None, 0, None, None) == 0
    assert lib.woq_dequantize_int4_groups(None, None, None, 0, 256, 32, 0, None, None) == 0


def test_codec_argument_checks(lib):
    fake = ctypes.c_void_p(4096)
    assert woq.STATUS[lib.woq_pack_uint4(fake, 3, fake, None)] == "WOQ_ESHAPE"
    assert woq.STATUS[lib.woq_unpack_uint4(fake, -2, fake, None)] == "WOQ_EINVAL"
    assert woq.STATUS[lib.woq_quantize_groups(fake, 2, 10, 4, 0, fake, fake, fake, None)] == "WOQ_EGROUP"
    assert woq.STATUS[lib.woq_quantize_groups(fake, 2, 8, 4, 2, fake, fake, fake, None)] == "WOQ_EINVAL"
    assert woq.STATUS[lib.woq_quantize_groups(None, 2, 8, 4, 0, fake, fake, fake, None)] == "WOQ_EINVAL"
    assert woq.STATUS[lib.woq_dequantize_int4_groups(fake, fake, fake, 2, 12, 3, 0, fake, None)] == "WOQ_EGROUP"
    assert woq.STATUS[lib.woq_dequantize_int4_groups(fake, fake, fake, 2, 12, 4, 5, fake, None)] == "WOQ_EINVAL"
    assert woq.STATUS[lib.woq_dequantize_int4_groups(fake, fake, None, 2, 12, 4, 0, fake, None)] == "WOQ_EINVAL"


def test_plan_buffer_checks(lib):
    assert woq.STATUS[lib.woq_linear_plan(1, 64, 256, 32, 0, None, 16)] == "WOQ_EINVAL"
    buf = ctypes.create_string_buffer(8)
    assert lib.woq_linear_plan(1, 64, 256, 32, 0, buf, len(buf)) == 0
    assert len(buf.value) == 7          # truncated, NUL-terminated


def test_prepared_layout_host_checks(lib):
    import oracle
    for n, k in ((0, 0), (1, 32), (17, 96), (4096, 4096), (14336, 4096), (5, 4160)):
        assert lib.woq_prepared_bytes(n, k) == oracle.prepared_bytes(n, k)
    assert lib.woq_prepared_bytes(4, 48) == 0          # k not a multiple of 32
    assert lib.woq_prepared_bytes(-1, 64) == 0
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    for fn in (lib.woq_prepare_int4, lib.woq_unprepare_int4):
        assert woq.STATUS[fn(fake, 4, 48, fake, None)] == "WOQ_ESHAPE"
        assert woq.STATUS[fn(fake, -1, 64, fake, None)] == "WOQ_EINVAL"
        assert woq.STATUS[fn(None, 4, 64, fake, None)] == "WOQ_EINVAL"
        assert woq.STATUS[fn(odd, 4, 64, fake, None)] == "WOQ_EALIGN"
        assert woq.STATUS[fn(fake, 1 << 31, 64, fake, None)] == "WOQ_EUNSUPPORTED"
        assert fn(None, 0, 64, None, None) == 0
    # the prepared linear shares the canonical one's checks
    rc = lib.woq_linear_int4_groups_prepared(fake, 1, odd, fake, fake, None, None, 64, 256, 32, 1,
                                             fake, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EALIGN"
    rc = lib.woq_linear_int4_groups_prepared(fake, 1, fake, fake, fake, None, None, 64, 256, 48, 1,
                                             fake, None, 0, None)
    assert woq.STATUS[rc] == "WOQ_EGROUP"


def test_signed_format_entry_points_validate_first(lib):
    fake = ctypes.c_void_p(1 << 20)    # never dereferenced: validation fails first
    odd = ctypes.c_void_p((1 << 20) + 8)
    st = lambda rc: woq.STATUS[rc]
    assert st(lib.woq_quantize_int4_sym_f16(fake, 4, 96, 3, fake, fake, None)) == "WOQ_EGROUP"
    assert st(lib.woq_quantize_int4_sym_f16(fake, 4, 96, 5, fake, fake, None)) == "WOQ_EGROUP"
    assert st(lib.woq_quantize_int4_sym_f16(None, 4, 96, 32, fake, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_quantize_int4_sym_f16(fake, 0, 96, 32, None, None, None)) == "WOQ_OK"
    assert st(lib.woq_pack_int4(fake, 7, fake, None)) == "WOQ_ESHAPE"
    assert st(lib.woq_pack_int4(None, 8, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_unpack_int4(fake, 7, fake, None)) == "WOQ_ESHAPE"
    assert st(lib.woq_dequantize_int4_sym_f16(fake, fake, 4, 64, 32, 7, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_dequantize_int4_sym_f16(fake, fake, 4, 64, 24, 0, fake, None)) == "WOQ_EGROUP"
    # the linear: missing scale, misaligned scale, empty problem, unsupported group
    assert st(lib.woq_linear_int4_sym_f16(fake, 1, fake, None, None, None, 64, 256, 32, 1,
                                          fake, None, 0, None)) == "WOQ_EINVAL"
    assert st(lib.woq_linear_int4_sym_f16(fake, 1, fake, odd, None, None, 64, 256, 32, 1,
                                          fake, None, 0, None)) == "WOQ_EALIGN"
    assert st(lib.woq_linear_int4_sym_f16(fake, 0, fake, fake, None, None, 64, 256, 32, 1,
                                          fake, None, 0, None)) == "WOQ_OK"
    assert st(lib.woq_linear_int4_sym_f16(fake, 1, fake, fake, None, None, 64, 256, 16, 1,
                                          fake, None, 0, None)) == "WOQ_EUNSUPPORTED"
    assert st(lib.woq_linear_int4_sym_f16_prepared(fake, 1, fake, None, None, None, 64, 256, 32,
                                                   1, fake, None, 0, None)) == "WOQ_EINVAL"


def test_mxfp4_entry_points_validate_first(lib):
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    st = lambda rc: woq.STATUS[rc]
    assert st(lib.woq_quantize_mxfp4(fake, 4, 48, fake, fake, None)) == "WOQ_EGROUP"
    assert st(lib.woq_quantize_mxfp4(None, 4, 64, fake, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_quantize_mxfp4(fake, 0, 64, None, None, None)) == "WOQ_OK"
    assert st(lib.woq_dequantize_mxfp4(fake, fake, 4, 64, 9, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_dequantize_mxfp4(fake, fake, 4, 40, 0, fake, None)) == "WOQ_EGROUP"
    assert st(lib.woq_linear_mxfp4(fake, 1, fake, None, None, 64, 256, 1, fake, None, 0, None)) == "WOQ_EINVAL"
    assert st(lib.woq_linear_mxfp4(fake, 1, fake, odd, None, 64, 256, 1, fake, None, 0, None)) == "WOQ_EALIGN"
    assert st(lib.woq_linear_mxfp4(fake, 1, fake, fake, None, 64, 48, 1, fake, None, 0, None)) == "WOQ_EGROUP"
    assert st(lib.woq_linear_mxfp4(fake, 0, fake, fake, None, 64, 256, 1, fake, None, 0, None)) == "WOQ_OK"


def test_int4_rows_entry_points_validate_first(lib):
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    st = lambda rc: woq.STATUS[rc]
    assert st(lib.woq_quantize_int4_rows(fake, 4, 7, fake, fake, None)) == "WOQ_ESHAPE"
    assert st(lib.woq_quantize_int4_rows(None, 4, 8, fake, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_quantize_int4_rows(fake, 0, 8, None, None, None)) == "WOQ_OK"
    assert st(lib.woq_dequantize_int4_rows(fake, fake, 4, 8, 5, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_linear_int4_rows(fake, 1, fake, None, None, None, 64, 256, 1, fake, None, 0, None)) == "WOQ_EINVAL"
    assert st(lib.woq_linear_int4_rows(fake, 1, fake, odd, None, None, 64, 256, 1, fake, None, 0, None)) == "WOQ_EALIGN"
    assert st(lib.woq_linear_int4_rows(fake, 1, fake, fake, None, None, 64, 250, 1, fake, None, 0, None)) == "WOQ_EUNSUPPORTED"
    assert st(lib.woq_linear_int4_rows(fake, 1, fake, fake, None, None, 64, 251, 1, fake, None, 0, None)) == "WOQ_ESHAPE"
    assert st(lib.woq_linear_int4_rows(fake, 0, fake, fake, None, None, 64, 256, 1, fake, None, 0, None)) == "WOQ_OK"
    # the row layout runs in the largest supported group dividing k
    assert lib.woq_linear_int4_rows_workspace_bytes(256, 512, 4096, 0) == lib.woq_linear_workspace_bytes(256, 512, 4096, 256, 0)
    assert lib.woq_linear_int4_rows_workspace_bytes(256, 512, 96, 0) == lib.woq_linear_workspace_bytes(256, 512, 96, 32, 0)


def test_gptq_entry_point_validates_first(lib):
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 1)
    st = lambda rc: woq.STATUS[rc]
    args = lambda **kw: [kw.get("w", fake), kw.get("x", fake), kw.get("t", 16), kw.get("n", 8), kw.get("k", 256),
                         kw.get("group", 128), kw.get("act", 0), kw.get("damp", 0.01), fake, fake, fake,
                         kw.get("order", None), None]
    assert st(lib.woq_gptq_quantize(*args(group=96))) == "WOQ_EGROUP"
    assert st(lib.woq_gptq_quantize(*args(group=0))) == "WOQ_EGROUP"
    assert st(lib.woq_gptq_quantize(*args(k=512, group=512))) == "WOQ_EUNSUPPORTED"
    assert st(lib.woq_gptq_quantize(*args(act=1))) == "WOQ_EINVAL"              # order missing
    assert st(lib.woq_gptq_quantize(*args(act=2, order=fake))) == "WOQ_EINVAL"
    assert st(lib.woq_gptq_quantize(*args(damp=float("nan")))) == "WOQ_EINVAL"
    assert st(lib.woq_gptq_quantize(*args(damp=-1.0))) == "WOQ_EINVAL"
    assert st(lib.woq_gptq_quantize(*args(x=None))) == "WOQ_EINVAL"
    assert st(lib.woq_gptq_quantize(*args(w=odd))) == "WOQ_EALIGN"
    assert st(lib.woq_gptq_quantize(*args(n=-1))) == "WOQ_EINVAL"
    assert st(lib.woq_gptq_quantize(*args(n=0))) == "WOQ_OK"
    assert st(lib.woq_gptq_quantize(*args(k=0))) == "WOQ_OK"


def test_awq_entry_point_validates_first(lib):
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 2)
    best = ctypes.c_int32(-1)
    st = lambda rc: woq.STATUS[rc]
    args = lambda **kw: [kw.get("w", fake), fake, kw.get("t", 16), kw.get("n", 8), kw.get("k", 256),
                         kw.get("group", 128), kw.get("grid", 20), fake, fake, fake, kw.get("s", fake),
                         kw.get("losses", None), ctypes.byref(best), None]
    assert st(lib.woq_awq_search(*args(t=0))) == "WOQ_EINVAL"
    assert st(lib.woq_awq_search(*args(grid=0))) == "WOQ_EINVAL"
    assert st(lib.woq_awq_search(*args(grid=1001))) == "WOQ_EINVAL"
    assert st(lib.woq_awq_search(*args(group=96))) == "WOQ_EGROUP"
    assert st(lib.woq_awq_search(*args(s=None))) == "WOQ_EINVAL"
    assert st(lib.woq_awq_search(*args(w=odd))) == "WOQ_EALIGN"
    assert st(lib.woq_awq_search(*args(losses=odd))) == "WOQ_EALIGN"
    assert st(lib.woq_awq_search(*args(n=0))) == "WOQ_OK"
    assert best.value == -1


def test_zero_point_entry_points_validate_first(lib, monkeypatch):
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    st = lambda rc: woq.STATUS[rc]
    assert st(lib.woq_pack_zero_points(None, 4, 8, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_pack_zero_points(fake, -1, 8, fake, None)) == "WOQ_EINVAL"
    assert st(lib.woq_pack_zero_points(fake, 0, 8, None, None)) == "WOQ_OK"
    assert st(lib.woq_unpack_zero_points(fake, 4, 8, None, None)) == "WOQ_EINVAL"
    assert st(lib.woq_unpack_zero_points(None, 4, 0, None, None)) == "WOQ_OK"
    ws = lib.woq_linear_int4_groups_zp4_workspace_bytes
    # the kernels read packed zero points as they are: the linear's own workspace ...
    assert ws(1, 4096, 4096, 128, 0) == lib.woq_linear_workspace_bytes(1, 4096, 4096, 128, 0) == 0
    assert ws(256, 300, 4096, 64, 1) == lib.woq_linear_workspace_bytes(256, 300, 4096, 64, 1)
    assert ws(16, 300, 4096, 64, 1) == lib.woq_linear_workspace_bytes(16, 300, 4096, 64, 1)
    # ... except on the tile GEMV (m <= 4 with WOQ_DECODE_MFMA set), which takes them unpacked
    # (n * k/group bytes, rounded up to 256)
    monkeypatch.setenv("WOQ_DECODE_MFMA", "1")
    assert ws(1, 300, 4096, 128, 0) == (300 * 32 + 255) // 256 * 256 + lib.woq_linear_workspace_bytes(
        1, 300, 4096, 128, 0)
    monkeypatch.delenv("WOQ_DECODE_MFMA")
    assert ws(0, 4096, 4096, 128, 0) == 0 and ws(1, 4096, 4000, 128, 0) == 0
    zp4 = lambda **kw: lib.woq_linear_int4_groups_zp4(fake, 200, fake, fake, kw.get("zp", fake), None, None, 64,
                                                      256, 128, 1, fake, kw.get("ws", fake), kw.get("wsb", 1 << 20),
                                                      None)
    assert st(zp4(zp=None)) == "WOQ_EINVAL"
    assert st(zp4(ws=None, wsb=0)) == "WOQ_EWORKSPACE"
    assert st(zp4(wsb=16)) == "WOQ_EWORKSPACE"
    assert st(zp4(ws=odd)) == "WOQ_EALIGN"
