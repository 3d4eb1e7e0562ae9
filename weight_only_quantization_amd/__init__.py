"""Group-wise 4-bit weight-only linear layers on MI355X (gfx950).

Thin Python binding of ``libwoq.so`` (C ABI declared in ``include/woq.h``).
Every function here only marshals arguments: it checks that tensors live on
the GPU with the expected dtype, allocates outputs and workspace with
PyTorch, and passes raw device pointers plus the current HIP stream to the
library.  All arithmetic runs in the library's HIP kernels; there is no
fallback path, and a missing or unloadable library raises.

Names follow the std.quant functions of the linnet docs "Quantization" page:
``quantize_groups``, ``pack_uint4``, ``unpack_uint4``,
``dequantize_int4_groups``, ``linear_int4_groups`` (C names carry a ``woq_``
prefix).
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path
from typing import Optional

import torch  # loads the HIP runtime that libwoq.so then binds to

__all__ = [
    "WoqError",
    "load",
    "library_path",
    "quantize_groups",
    "gptq_quantize",
    "pack_zero_points",
    "unpack_zero_points",
    "linear_int4_groups_zp4",
    "awq_search",
    "pack_uint4",
    "unpack_uint4",
    "dequantize_int4_groups",
    "linear_int4_groups",
    "linear_int4_groups_prepared",
    "linear_int4_groups_grouped",
    "prepare_int4",
    "unprepare_int4",
    "prepared_bytes",
    "linear_workspace_bytes",
    "linear_plan",
    "quantize_int4_sym",
    "pack_int4",
    "unpack_int4",
    "dequantize_int4_sym",
    "linear_int4_sym",
    "quantize_int4_rows",
    "dequantize_int4_rows",
    "linear_int4_rows",
    "quantize_mxfp4",
    "dequantize_mxfp4",
    "linear_mxfp4",
    "STATUS",
]

_PKG = Path(__file__).resolve().parent
_LIB: Optional[ctypes.CDLL] = None

STATUS = {
    0: "WOQ_OK", 1: "WOQ_EINVAL", 2: "WOQ_ESHAPE", 3: "WOQ_EGROUP", 4: "WOQ_ENONFINITE",
    5: "WOQ_ERANGE", 6: "WOQ_EWORKSPACE", 7: "WOQ_EUNSUPPORTED", 8: "WOQ_EALIGN", 9: "WOQ_EHIP",
    10: "WOQ_ENOTPD",
}
F32, BF16 = 0, 1


class WoqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = _LIB.woq_status_str(status).decode() if _LIB is not None else ""
        super().__init__(f"{where}: {self.name} ({msg})")


def library_path() -> Path:
    return Path(os.environ.get("WOQ_LIBRARY", _PKG / "libwoq.so"))


def load() -> ctypes.CDLL:
    """Load libwoq.so (once).  Raises if it is missing: there is no fallback."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not path.exists():
        raise ImportError(f"{path} is missing; build it with __graft_entry__.build() "
                          "or python weight_only_quantization_amd/_build.py")
    lib = ctypes.CDLL(str(path))
    c_i32, c_i64, c_p, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "woq_status_str": (ctypes.c_char_p, [c_i32]),
        "woq_version": (c_i32, []),
        "woq_quantize_groups": (c_i32, [c_p, c_i64, c_i64, c_i32, c_i32, c_p, c_p, c_p, c_p]),
        "woq_pack_uint4": (c_i32, [c_p, c_i64, c_p, c_p]),
        "woq_unpack_uint4": (c_i32, [c_p, c_i64, c_p, c_p]),
        "woq_dequantize_int4_groups": (c_i32, [c_p, c_p, c_p, c_i64, c_i64, c_i32, c_i32, c_p, c_p]),
        "woq_linear_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32, c_i32]),
        "woq_linear_int4_groups": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64,
                                           c_i32, c_i32, c_p, c_p, c_sz, c_p]),
        "woq_linear_plan": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, ctypes.c_char_p, c_sz]),
        "woq_prepared_bytes": (c_sz, [c_i64, c_i64]),
        "woq_prepare_int4": (c_i32, [c_p, c_i64, c_i64, c_p, c_p]),
        "woq_unprepare_int4": (c_i32, [c_p, c_i64, c_i64, c_p, c_p]),
        "woq_linear_int4_groups_prepared": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64,
                                                    c_i32, c_i32, c_p, c_p, c_sz, c_p]),
        "woq_linear_int4_groups_grouped": (c_i32, [c_p, c_i64, c_i32, c_p, c_p, c_p, c_p, c_p, c_i64,
                                                   c_i32, c_i32, c_i32, c_p, c_p, c_sz, c_p]),
        "woq_quantize_int4_sym_f16": (c_i32, [c_p, c_i64, c_i64, c_i32, c_p, c_p, c_p]),
        "woq_pack_int4": (c_i32, [c_p, c_i64, c_p, c_p]),
        "woq_unpack_int4": (c_i32, [c_p, c_i64, c_p, c_p]),
        "woq_dequantize_int4_sym_f16": (c_i32, [c_p, c_p, c_i64, c_i64, c_i32, c_i32, c_p, c_p]),
        "woq_linear_int4_sym_f16": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i32,
                                            c_i32, c_p, c_p, c_sz, c_p]),
        "woq_linear_int4_sym_f16_prepared": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_p, c_i64, c_i64,
                                                     c_i32, c_i32, c_p, c_p, c_sz, c_p]),
        "woq_quantize_mxfp4": (c_i32, [c_p, c_i64, c_i64, c_p, c_p, c_p]),
        "woq_quantize_int4_rows": (c_i32, [c_p, c_i64, c_i64, c_p, c_p, c_p]),
        "woq_dequantize_int4_rows": (c_i32, [c_p, c_p, c_i64, c_i64, c_i32, c_p, c_p]),
        "woq_linear_int4_rows_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
        "woq_linear_int4_rows": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i32, c_p, c_p,
                                         c_sz, c_p]),
        "woq_dequantize_mxfp4": (c_i32, [c_p, c_p, c_i64, c_i64, c_i32, c_p, c_p]),
        "woq_linear_mxfp4": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_i64, c_i64, c_i32, c_p, c_p, c_sz,
                                     c_p]),
        "woq_gptq_quantize": (c_i32, [c_p, c_p, c_i64, c_i64, c_i64, c_i32, c_i32, ctypes.c_double, c_p, c_p,
                                      c_p, c_p, c_p]),
        "woq_awq_search": (c_i32, [c_p, c_p, c_i64, c_i64, c_i64, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_p,
                                   c_p]),
        "woq_pack_zero_points": (c_i32, [c_p, c_i64, c_i64, c_p, c_p]),
        "woq_unpack_zero_points": (c_i32, [c_p, c_i64, c_i64, c_p, c_p]),
        "woq_linear_int4_groups_zp4": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i32, c_i32,
                                               c_p, c_p, c_sz, c_p]),
        "woq_linear_int4_groups_zp4_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32, c_i32]),
        "woq_linear_noalloc_max_workspace_bytes": (c_sz, []),
        "woq_linear_int4_groups_noalloc": (c_i32, [c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i32, c_i32,
                                                   c_p, c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise WoqError(status, where)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype: torch.dtype, name: str, gpu: bool = True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if gpu and not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_sizes(m: int, n: int, k: int, *, sized=(), bias=None, order=None, out=None):
    """Every operand must hold exactly what the kernels address for (m, n, k).

    The kernels size their buffer descriptors from these numbers, not from the
    allocations, so a short tensor would be read or written out of bounds on the
    device: refuse it here instead.  ``sized`` lists (name, tensor, elements).
    """
    for name, t, numel in sized:
        if t is not None and t.numel() != numel:
            raise ValueError(f"{name} holds {t.numel()} elements, expected {numel} for [{n}, {k}]")
    if bias is not None and bias.numel() != n:
        raise ValueError(f"bias holds {bias.numel()} elements, expected N = {n}")
    if order is not None and order.numel() != k:
        raise ValueError(f"order holds {order.numel()} elements, expected K = {k}")
    if out is not None and tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}], got {list(out.shape)}")


def _on_gpu(x: torch.Tensor, **named):
    """x on the GPU, and every other named tensor (None skipped) on x's device."""
    if not x.is_cuda:
        raise ValueError("x must be on the GPU")
    for name, t in named.items():
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} must be on x's device ({x.device}), got {t.device}")


def _groups(k: int, group: int) -> int:
    """Groups per row, or 0 when the group size is invalid (the library then
    reports it without touching memory)."""
    return k // group if group > 0 and k % group == 0 else 0


def quantize_groups(w: torch.Tensor, group: int = 128, symmetric: bool = False):
    """Round-to-nearest group quantizer on the GPU.

    w: float32 [N, K].  Returns (q uint8 [N, K] codes 0..15, scale float32
    [N, K/group], zero uint8 [N, K/group]).  Synchronizes the current stream.
    """
    lib = load()
    _need(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    ng = k // group if group > 0 else 0
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n, ng), dtype=torch.float32, device=w.device)
    zero = torch.empty((n, ng), dtype=torch.uint8, device=w.device)
    _check(lib.woq_quantize_groups(_ptr(w), n, k, group, int(bool(symmetric)), _ptr(q),
                                   _ptr(scale), _ptr(zero), _stream()), "quantize_groups")
    return q, scale, zero


def gptq_quantize(w: torch.Tensor, x: Optional[torch.Tensor], group: int = 128, act_order: bool = False,
                  damp: float = 0.01):
    """GPTQ of one layer on the GPU, in float64.

    w: float32 [N, K]; x: bfloat16 calibration inputs [T, K] (None for none).
    Returns (q uint8 [N, K], scale float32 [N, K/group], zero uint8
    [N, K/group], order int32 [K] or None), the columns in visiting order; pass
    `order` to the linear calls.  Synchronizes the current stream.
    """
    lib = load()
    _need(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    t = 0
    if x is not None:
        _need(x, torch.bfloat16, "x")
        if x.dim() != 2 or x.shape[1] != k:
            raise ValueError("x must be [T, K]")
        t = x.shape[0]
    ng = k // group if group > 0 else 0
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n, ng), dtype=torch.float32, device=w.device)
    zero = torch.empty((n, ng), dtype=torch.uint8, device=w.device)
    order = torch.empty((k,), dtype=torch.int32, device=w.device) if act_order else None
    _check(lib.woq_gptq_quantize(_ptr(w), _ptr(x), t, n, k, group, int(bool(act_order)), float(damp), _ptr(q),
                                 _ptr(scale), _ptr(zero), _ptr(order), _stream()), "gptq_quantize")
    return q, scale, zero, order


def awq_search(w: torch.Tensor, x: torch.Tensor, group: int = 128, n_grid: int = 20):
    """AWQ scale search for one layer on the GPU.

    w: float32 [N, K]; x: bfloat16 calibration inputs [T, K], T >= 1.  Returns
    (q uint8 [N, K], scale float32 [N, K/group], zero uint8 [N, K/group]) of the
    scaled weights W diag(s), s float32 [K], the chosen grid index (alpha =
    index / n_grid) and the error of every grid point (float64 [n_grid + 1]).
    The layer then computes with x / s.  Synchronizes the current stream.
    """
    lib = load()
    _need(w, torch.float32, "w")
    _need(x, torch.bfloat16, "x")
    if w.dim() != 2 or x.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("w must be [N, K] and x [T, K]")
    n, k = w.shape
    ng = k // group if group > 0 else 0
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n, ng), dtype=torch.float32, device=w.device)
    zero = torch.empty((n, ng), dtype=torch.uint8, device=w.device)
    s = torch.empty((k,), dtype=torch.float32, device=w.device)
    losses = torch.empty((max(n_grid, 0) + 1,), dtype=torch.float64, device=w.device)
    best = ctypes.c_int32(-1)
    _check(lib.woq_awq_search(_ptr(w), _ptr(x), x.shape[0], n, k, group, n_grid, _ptr(q), _ptr(scale),
                              _ptr(zero), _ptr(s), _ptr(losses), ctypes.byref(best), _stream()), "awq_search")
    return q, scale, zero, s, best.value, losses


def pack_uint4(q: torch.Tensor) -> torch.Tensor:
    """uint8 codes [..., 2c] -> packed bytes [..., c] (even element in the low nibble)."""
    lib = load()
    _need(q, torch.uint8, "q")
    if q.shape[-1] % 2:
        raise ValueError("last dimension must be even")
    out = torch.empty(q.shape[:-1] + (q.shape[-1] // 2,), dtype=torch.uint8, device=q.device)
    _check(lib.woq_pack_uint4(_ptr(q), q.numel(), _ptr(out), _stream()), "pack_uint4")
    return out


def unpack_uint4(packed: torch.Tensor) -> torch.Tensor:
    """packed bytes [..., c] -> uint8 codes [..., 2c]."""
    lib = load()
    _need(packed, torch.uint8, "packed")
    out = torch.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=torch.uint8,
                      device=packed.device)
    _check(lib.woq_unpack_uint4(_ptr(packed), out.numel(), _ptr(out), _stream()), "unpack_uint4")
    return out


def _weight_dims(packed: torch.Tensor, scale: torch.Tensor, group: Optional[int]):
    n = packed.shape[0]
    k = 2 * (packed.numel() // n) if n else 0
    if group is None:
        if scale.dim() != 2 or scale.shape[1] == 0:
            raise ValueError("cannot infer the group size from scale")
        group = k // scale.shape[1]
    return n, k, int(group)


def dequantize_int4_groups(packed: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor,
                           group: Optional[int] = None,
                           out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """(q - zero) * scale per group -> [N, K] float32 or bfloat16."""
    lib = load()
    _need(packed, torch.uint8, "packed")
    _need(scale, torch.float32, "scale")
    _need(zero, torch.uint8, "zero")
    n, k, group = _weight_dims(packed, scale, group)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    out = torch.empty((n, k), dtype=out_dtype, device=packed.device)
    _check(lib.woq_dequantize_int4_groups(_ptr(packed), _ptr(scale), _ptr(zero), n, k, group,
                                          F32 if out_dtype == torch.float32 else BF16, _ptr(out),
                                          _stream()), "dequantize_int4_groups")
    return out


def linear_workspace_bytes(m: int, n: int, k: int, group: int, has_order: bool) -> int:
    return int(load().woq_linear_workspace_bytes(m, n, k, group, int(bool(has_order))))


def linear_plan(m: int, n: int, k: int, group: int, has_order: bool = False) -> str:
    """The kernel plan the library uses for these sizes (a one-line description)."""
    lib = load()
    buf = ctypes.create_string_buffer(512)
    _check(lib.woq_linear_plan(m, n, k, group, int(bool(has_order)), buf, len(buf)), "linear_plan")
    return buf.value.decode()


def prepared_bytes(n: int, k: int) -> int:
    """Bytes of the prepared (fragment-ordered) layout of an [n, k] weight."""
    return int(load().woq_prepared_bytes(n, k))


def prepare_int4(packed: torch.Tensor, k: Optional[int] = None) -> torch.Tensor:
    """Canonical packed rows [N, K/2] (or [N, K/G, G/2]) -> prepared uint8 buffer.

    The layout is the one ``woq_prepare_int4`` documents: 1 KB blocks of 16
    outputs x 128 inputs in MFMA operand order.  Asynchronous.
    """
    lib = load()
    _need(packed, torch.uint8, "packed")
    n = packed.shape[0]
    kk = 2 * (packed.numel() // n) if n else (k or 0)
    k = kk if k is None else k
    if k != kk:
        raise ValueError(f"packed holds {kk} inputs per row, not {k}")
    out = torch.empty(max(prepared_bytes(n, k), 1), dtype=torch.uint8, device=packed.device)
    _check(lib.woq_prepare_int4(_ptr(packed), n, k, _ptr(out), _stream()), "prepare_int4")
    return out[:prepared_bytes(n, k)]


def unprepare_int4(prepared: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """Inverse of :func:`prepare_int4`: prepared buffer -> packed rows [N, K/2]."""
    lib = load()
    _need(prepared, torch.uint8, "prepared")
    if prepared.numel() < prepared_bytes(n, k):
        raise ValueError("prepared buffer is smaller than the layout of [n, k]")
    out = torch.empty((n, k // 2), dtype=torch.uint8, device=prepared.device)
    _check(lib.woq_unprepare_int4(_ptr(prepared), n, k, _ptr(out), _stream()), "unprepare_int4")
    return out


def linear_int4_groups_prepared(x: torch.Tensor, prepared: torch.Tensor, scale: torch.Tensor,
                                zero: torch.Tensor, bias: Optional[torch.Tensor] = None,
                                order: Optional[torch.Tensor] = None,
                                out_dtype: torch.dtype = torch.bfloat16,
                                out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """:func:`linear_int4_groups` over prepared weights (see :func:`prepare_int4`).

    N comes from scale [N, K/G], K from x [M, K], the group from both.
    """
    _need(scale, torch.float32, "scale", gpu=False)
    if x.dim() != 2 or scale.dim() != 2 or scale.shape[1] == 0:
        raise ValueError("x must be [M, K] and scale [N, K/G]")
    n, k = scale.shape[0], x.shape[1]
    if prepared.numel() < prepared_bytes(n, k):
        raise ValueError("prepared buffer is smaller than the layout of [n, k]")
    return _linear(x, prepared, scale, zero, bias, order, n, k, k // scale.shape[1], out_dtype,
                   out, workspace, True)


def linear_int4_groups(x: torch.Tensor, packed: torch.Tensor, scale: torch.Tensor,
                       zero: torch.Tensor, bias: Optional[torch.Tensor] = None,
                       order: Optional[torch.Tensor] = None, group: Optional[int] = None,
                       out_dtype: torch.dtype = torch.bfloat16,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x' . dequant(W)^T + bias with x' = x[:, order] when order is given.

    x: bfloat16 [M, K]; packed uint8 [N, K/2] (or [N, K/G, G/2]); scale float32
    [N, K/G]; zero uint8 [N, K/G]; bias float32 [N] or None; order int32 [K] or
    None.  Returns y [M, N] of out_dtype (bfloat16 or float32).  Asynchronous
    on the current stream.
    """
    _need(packed, torch.uint8, "packed", gpu=False)
    _need(scale, torch.float32, "scale", gpu=False)
    n, k, group = _weight_dims(packed, scale, group)
    if x.dim() == 2 and x.shape[1] != k:
        raise ValueError(f"x has {x.shape[1]} inputs, the weight {k}")
    return _linear(x, packed, scale, zero, bias, order, n, k, group, out_dtype, out, workspace,
                   False)


def _linear(x, weights, scale, zero, bias, order, n, k, group, out_dtype, out, workspace,
            prepared: bool, sym16: bool = False):
    lib = load()
    _need(x, torch.bfloat16, "x", gpu=False)
    _need(weights, torch.uint8, "prepared" if prepared else "packed", gpu=False)
    if sym16:
        _need(scale, torch.float16, "scale", gpu=False)
    else:
        _need(scale, torch.float32, "scale", gpu=False)
        _need(zero, torch.uint8, "zero", gpu=False)
    if bias is not None:
        _need(bias, torch.float32, "bias", gpu=False)
    if order is not None:
        _need(order, torch.int32, "order", gpu=False)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [M, {k}]")
    m = x.shape[0]
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    if out is not None:
        _need(out, out_dtype, "out", gpu=False)
    ng = _groups(k, group)
    sized = [("scale", scale, n * ng), ("zero", zero, n * ng)] if ng else []
    if not prepared:
        sized.append(("packed", weights, n * (k // 2)))
    elif weights.numel() < prepared_bytes(n, k):
        raise ValueError("prepared buffer is smaller than the layout of [n, k]")
    _check_sizes(m, n, k, sized=sized, bias=bias, order=order, out=out)
    _on_gpu(x, weights=weights, scale=scale, zero=zero, bias=bias, order=order, out=out,
            workspace=workspace)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    need = int(lib.woq_linear_workspace_bytes(m, n, k, group, int(order is not None)))
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() if (need and workspace is not None) else 0
    y_dtype = F32 if out_dtype == torch.float32 else BF16
    ws_ptr = _ptr(workspace) if need else None
    if sym16:
        fn = lib.woq_linear_int4_sym_f16_prepared if prepared else lib.woq_linear_int4_sym_f16
        _check(fn(_ptr(x), m, _ptr(weights), _ptr(scale), _ptr(bias), _ptr(order), n, k, group,
                  y_dtype, _ptr(out), ws_ptr, wsb, _stream()),
               "linear_int4_sym_f16_prepared" if prepared else "linear_int4_sym_f16")
        return out
    fn = lib.woq_linear_int4_groups_prepared if prepared else lib.woq_linear_int4_groups
    _check(fn(_ptr(x), m, _ptr(weights), _ptr(scale), _ptr(zero), _ptr(bias), _ptr(order), n, k,
              group, y_dtype, _ptr(out), ws_ptr, wsb, _stream()),
           "linear_int4_groups_prepared" if prepared else "linear_int4_groups")
    return out


# ---------------------------------------------------------------------------
# Packed 4-bit zero points (the MatMulNBits layout)
# ---------------------------------------------------------------------------

def pack_zero_points(zero: torch.Tensor) -> torch.Tensor:
    """zero uint8 [N, G_n] (0..15) -> [N, ceil(G_n / 2)], group 2j in the low nibble.  Syncs."""
    lib = load()
    _need(zero, torch.uint8, "zero")
    if zero.dim() != 2:
        raise ValueError("zero must be [N, groups]")
    n, ng = zero.shape
    out = torch.empty((n, (ng + 1) // 2), dtype=torch.uint8, device=zero.device)
    _check(lib.woq_pack_zero_points(_ptr(zero), n, ng, _ptr(out), _stream()), "pack_zero_points")
    return out


def unpack_zero_points(zero_packed: torch.Tensor, ngroups: int) -> torch.Tensor:
    """Inverse of pack_zero_points: [N, ceil(G_n / 2)] -> uint8 [N, G_n].  Asynchronous."""
    lib = load()
    _need(zero_packed, torch.uint8, "zero_packed")
    if zero_packed.dim() != 2 or zero_packed.shape[1] != (ngroups + 1) // 2:
        raise ValueError("zero_packed must be [N, ceil(ngroups / 2)]")
    n = zero_packed.shape[0]
    out = torch.empty((n, ngroups), dtype=torch.uint8, device=zero_packed.device)
    _check(lib.woq_unpack_zero_points(_ptr(zero_packed), n, ngroups, _ptr(out), _stream()), "unpack_zero_points")
    return out


def linear_int4_groups_zp4_workspace_bytes(m: int, n: int, k: int, group: int, has_order: bool) -> int:
    return int(load().woq_linear_int4_groups_zp4_workspace_bytes(m, n, k, group, int(bool(has_order))))


def linear_int4_groups_zp4(x: torch.Tensor, packed: torch.Tensor, scale: torch.Tensor,
                           zero_packed: torch.Tensor, bias: Optional[torch.Tensor] = None,
                           order: Optional[torch.Tensor] = None, group: Optional[int] = None,
                           out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """linear_int4_groups with packed 4-bit zero points [N, ceil(K/G / 2)].  Asynchronous."""
    lib = load()
    _need(x, torch.bfloat16, "x", gpu=False)
    _need(packed, torch.uint8, "packed", gpu=False)
    _need(scale, torch.float32, "scale", gpu=False)
    _need(zero_packed, torch.uint8, "zero_packed", gpu=False)
    if bias is not None:
        _need(bias, torch.float32, "bias", gpu=False)
    if order is not None:
        _need(order, torch.int32, "order", gpu=False)
    n, k, group = _weight_dims(packed, scale, group)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [M, K]")
    m = x.shape[0]
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    if out is not None:
        _need(out, out_dtype, "out", gpu=False)
    ng = _groups(k, group)
    _check_sizes(m, n, k, sized=[("scale", scale, n * ng), ("zero_packed", zero_packed, n * ((ng + 1) // 2))]
                 if ng else [], bias=bias, order=order, out=out)
    _on_gpu(x, packed=packed, scale=scale, zero_packed=zero_packed, bias=bias, order=order, out=out,
            workspace=workspace)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    need = int(lib.woq_linear_int4_groups_zp4_workspace_bytes(m, n, k, group, int(order is not None)))
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() if (need and workspace is not None) else 0
    _check(lib.woq_linear_int4_groups_zp4(_ptr(x), m, _ptr(packed), _ptr(scale), _ptr(zero_packed), _ptr(bias),
                                          _ptr(order), n, k, group, F32 if out_dtype == torch.float32 else BF16,
                                          _ptr(out), _ptr(workspace) if need else None, wsb, _stream()),
           "linear_int4_groups_zp4")
    return out


# ---------------------------------------------------------------------------
# Signed int4 groups with float16 scales (tinyllm L8.5, "int4 per group")
# ---------------------------------------------------------------------------

def quantize_int4_sym(w: torch.Tensor, group: int = 32):
    """Symmetric signed int4 per group with a float16 scale on the GPU.

    w: float32 [N, K].  Returns (codes int8 [N, K] in -8..7, scale float16
    [N, K/group]): s16 = float16(amax / 7), codes rint(w / s16).  Synchronizes.
    """
    lib = load()
    _need(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    ng = k // group if group > 0 else 0
    codes = torch.empty((n, k), dtype=torch.int8, device=w.device)
    scale = torch.empty((n, ng), dtype=torch.float16, device=w.device)
    _check(lib.woq_quantize_int4_sym_f16(_ptr(w), n, k, group, _ptr(codes), _ptr(scale), _stream()),
           "quantize_int4_sym_f16")
    return codes, scale


def pack_int4(codes: torch.Tensor) -> torch.Tensor:
    """int8 codes -8..7 [..., 2c] -> bytes [..., c], 4-bit two's complement, even element low."""
    lib = load()
    _need(codes, torch.int8, "codes")
    if codes.shape[-1] % 2:
        raise ValueError("last dimension must be even")
    out = torch.empty(codes.shape[:-1] + (codes.shape[-1] // 2,), dtype=torch.uint8, device=codes.device)
    _check(lib.woq_pack_int4(_ptr(codes), codes.numel(), _ptr(out), _stream()), "pack_int4")
    return out


def unpack_int4(packed: torch.Tensor) -> torch.Tensor:
    """bytes [..., c] -> int8 codes [..., 2c], each nibble sign-extended."""
    lib = load()
    _need(packed, torch.uint8, "packed")
    out = torch.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=torch.int8, device=packed.device)
    _check(lib.woq_unpack_int4(_ptr(packed), out.numel(), _ptr(out), _stream()), "unpack_int4")
    return out


def dequantize_int4_sym(packed: torch.Tensor, scale: torch.Tensor, group: Optional[int] = None,
                        out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """codes * float16 scale per group -> [N, K] float32 or bfloat16."""
    lib = load()
    _need(packed, torch.uint8, "packed")
    _need(scale, torch.float16, "scale")
    n, k, group = _weight_dims(packed, scale, group)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    out = torch.empty((n, k), dtype=out_dtype, device=packed.device)
    _check(lib.woq_dequantize_int4_sym_f16(_ptr(packed), _ptr(scale), n, k, group,
                                           F32 if out_dtype == torch.float32 else BF16, _ptr(out),
                                           _stream()), "dequantize_int4_sym_f16")
    return out


def linear_int4_sym(x: torch.Tensor, packed: torch.Tensor, scale: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None,
                    group: Optional[int] = None, out_dtype: torch.dtype = torch.bfloat16,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    prepared: bool = False) -> torch.Tensor:
    """y = x' . (codes * s16)^T + bias over signed int4 groups with float16 scales.

    x: bfloat16 [M, K]; packed uint8 [N, K/2] (or, with prepared=True, the
    buffer of :func:`prepare_int4`); scale float16 [N, K/G]; bias float32 [N] or
    None; order int32 [K] or None.  Asynchronous on the current stream.
    """
    _need(scale, torch.float16, "scale", gpu=False)
    if x.dim() != 2 or scale.dim() != 2 or scale.shape[1] == 0:
        raise ValueError("x must be [M, K] and scale [N, K/G]")
    n, k = scale.shape[0], x.shape[1]
    if prepared:
        if packed.numel() < prepared_bytes(n, k):
            raise ValueError("prepared buffer is smaller than the layout of [n, k]")
    elif packed.numel() != n * (k // 2):
        raise ValueError(f"packed holds {packed.numel()} bytes, expected {n * (k // 2)}")
    g = k // scale.shape[1] if group is None else group
    return _linear(x, packed, scale, None, bias, order, n, k, g, out_dtype, out, workspace,
                   prepared, sym16=True)


def linear_int4_groups_grouped(x: torch.Tensor, mats, prepared: bool = False,
                               out_dtype: torch.dtype = torch.bfloat16, outs=None,
                               workspace: Optional[torch.Tensor] = None):
    """Several linears over the same activations in one call.

    mats: 1..4 tuples (weights, scale, zero, bias or None), weights being packed
    rows [N_i, K/2] (or the prepared buffer when ``prepared``); all share x
    [M, K] and the group size.  Returns the list of y_i [M, N_i].  At M <= 4 the
    matrices share one kernel launch.  Asynchronous on the current stream.
    """
    lib = load()
    _need(x, torch.bfloat16, "x", gpu=False)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    if not 1 <= len(mats) <= 4:
        raise ValueError("between 1 and 4 matrices")
    m, k = x.shape
    group = None
    ns = []
    for i, (w, sc, z, b) in enumerate(mats):
        _need(w, torch.uint8, f"weights[{i}]", gpu=False)
        _need(sc, torch.float32, f"scale[{i}]", gpu=False)
        _need(z, torch.uint8, f"zero[{i}]", gpu=False)
        if b is not None:
            _need(b, torch.float32, f"bias[{i}]", gpu=False)
        if sc.dim() != 2 or sc.shape[1] == 0:
            raise ValueError("scale must be [N, K/G]")
        g = k // sc.shape[1]
        if group is not None and g != group:
            raise ValueError("all matrices must share the group size")
        group = g
        n_i = sc.shape[0]
        ns.append(n_i)
        ng = _groups(k, g)
        sized = [(f"scale[{i}]", sc, n_i * ng), (f"zero[{i}]", z, n_i * ng)] if ng else []
        if prepared:
            if w.numel() < prepared_bytes(n_i, k):
                raise ValueError(f"weights[{i}] hold fewer bytes than an [{n_i}, {k}] weight")
        else:
            sized.append((f"weights[{i}]", w, n_i * (k // 2)))
        _check_sizes(m, n_i, k, sized=sized, bias=b)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    made_outs = outs is None
    if outs is None:
        outs = [None] * len(mats)
    else:
        if len(outs) != len(mats):
            raise ValueError("one output per matrix")
        for i, o in enumerate(outs):
            _need(o, out_dtype, f"outs[{i}]", gpu=False)
            _check_sizes(m, ns[i], k, out=o)
    for i, (w, sc, z, b) in enumerate(mats):
        _on_gpu(x, **{f"weights_{i}": w, f"scale_{i}": sc, f"zero_{i}": z, f"bias_{i}": b,
                      f"outs_{i}": None if outs is None else outs[i]})
    _on_gpu(x, workspace=workspace)
    if made_outs:
        outs = [torch.empty((m, n), dtype=out_dtype, device=x.device) for n in ns]
    need = max(int(lib.woq_linear_workspace_bytes(m, n, k, group, 0)) for n in ns)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    cnt = len(mats)
    arr = lambda vals: (ctypes.c_void_p * cnt)(*vals)
    _check(lib.woq_linear_int4_groups_grouped(
        _ptr(x), m, cnt, arr([_ptr(w) for w, _, _, _ in mats]), arr([_ptr(sc) for _, sc, _, _ in mats]),
        arr([_ptr(z) for _, _, z, _ in mats]), arr([_ptr(b) for _, _, _, b in mats]),
        (ctypes.c_int64 * cnt)(*ns), k, group, int(bool(prepared)),
        F32 if out_dtype == torch.float32 else BF16, arr([_ptr(o) for o in outs]),
        _ptr(workspace) if need else None, workspace.numel() if need else 0, _stream()),
        "linear_int4_groups_grouped")
    return outs


# ---------------------------------------------------------------------------
# MXFP4: E2M1 codes in blocks of 32 with an E8M0 scale byte a block
# ---------------------------------------------------------------------------

def quantize_mxfp4(w: torch.Tensor):
    """MXFP4 quantizer on the GPU.  w: float32 [N, K], K a multiple of 32.

    Returns (codes uint8 [N, K] 0..15, scales uint8 [N, K/32] E8M0); pack the
    codes with :func:`pack_uint4`.  Synchronizes the current stream.
    """
    lib = load()
    _need(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 32), dtype=torch.uint8, device=w.device)
    _check(lib.woq_quantize_mxfp4(_ptr(w), n, k, _ptr(codes), _ptr(scales), _stream()), "quantize_mxfp4")
    return codes, scales


def dequantize_mxfp4(blocks: torch.Tensor, scales: torch.Tensor,
                     out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """E2M1 value * 2^(e - 127) -> [N, K] float32 or bfloat16 (K = 32 * scales.shape[1])."""
    lib = load()
    _need(blocks, torch.uint8, "blocks")
    _need(scales, torch.uint8, "scales")
    n, k = scales.shape[0], 32 * scales.shape[1]
    if blocks.numel() != n * k // 2:
        raise ValueError("blocks must hold N * K / 2 bytes")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    out = torch.empty((n, k), dtype=out_dtype, device=blocks.device)
    _check(lib.woq_dequantize_mxfp4(_ptr(blocks), _ptr(scales), n, k,
                                    F32 if out_dtype == torch.float32 else BF16, _ptr(out), _stream()),
           "dequantize_mxfp4")
    return out


def linear_mxfp4(x: torch.Tensor, blocks: torch.Tensor, scales: torch.Tensor,
                 bias: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x . dequant(W)^T + bias over MXFP4 weights.

    x: bfloat16 [M, K]; blocks uint8 [N, K/2] (or [N, K/32, 16]); scales uint8
    [N, K/32]; bias float32 [N] or None.  Asynchronous on the current stream.
    """
    lib = load()
    _need(x, torch.bfloat16, "x", gpu=False)
    _need(blocks, torch.uint8, "blocks", gpu=False)
    _need(scales, torch.uint8, "scales", gpu=False)
    if bias is not None:
        _need(bias, torch.float32, "bias", gpu=False)
    if x.dim() != 2 or scales.dim() != 2:
        raise ValueError("x must be [M, K] and scales [N, K/32]")
    m, k = x.shape
    n = scales.shape[0]
    if scales.shape[1] * 32 != k or blocks.numel() != n * k // 2:
        raise ValueError("blocks, scales and x disagree on K")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    if out is not None:
        _need(out, out_dtype, "out", gpu=False)
    _check_sizes(m, n, k, bias=bias, out=out)
    _on_gpu(x, blocks=blocks, scales=scales, bias=bias, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    need = int(lib.woq_linear_workspace_bytes(m, n, k, 32, 0))
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() if (need and workspace is not None) else 0
    _check(lib.woq_linear_mxfp4(_ptr(x), m, _ptr(blocks), _ptr(scales), _ptr(bias), n, k,
                                F32 if out_dtype == torch.float32 else BF16, _ptr(out),
                                _ptr(workspace) if need else None, wsb, _stream()), "linear_mxfp4")
    return out


# ---------------------------------------------------------------------------
# Int4Linear: signed int4 codes with one float32 scale a row
# ---------------------------------------------------------------------------

def quantize_int4_rows(w: torch.Tensor):
    """Symmetric signed int4 per row on the GPU: w float32 [N, K] -> (codes int8
    [N, K] in -8..7, scale float32 [N]); s = amax / 7, codes rint(w / s).  Syncs."""
    lib = load()
    _need(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.int8, device=w.device)
    scale = torch.empty((n,), dtype=torch.float32, device=w.device)
    _check(lib.woq_quantize_int4_rows(_ptr(w), n, k, _ptr(codes), _ptr(scale), _stream()),
           "quantize_int4_rows")
    return codes, scale


def dequantize_int4_rows(packed: torch.Tensor, scale: torch.Tensor,
                         out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """codes * scale[row] -> [N, K] float32 or bfloat16."""
    lib = load()
    _need(packed, torch.uint8, "packed")
    _need(scale, torch.float32, "scale")
    n = scale.shape[0]
    k = 2 * (packed.numel() // n) if n else 0
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    out = torch.empty((n, k), dtype=out_dtype, device=packed.device)
    _check(lib.woq_dequantize_int4_rows(_ptr(packed), _ptr(scale), n, k,
                                        F32 if out_dtype == torch.float32 else BF16, _ptr(out), _stream()),
           "dequantize_int4_rows")
    return out


def linear_int4_rows(x: torch.Tensor, packed: torch.Tensor, scale: torch.Tensor,
                     bias: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x' . (codes * scale[row])^T + bias over Int4Linear weights.

    x bfloat16 [M, K]; packed uint8 [N, K/2] of signed nibbles; scale float32
    [N]; bias float32 [N] or None; order int32 [K] or None.  Asynchronous.
    """
    lib = load()
    _need(x, torch.bfloat16, "x", gpu=False)
    _need(packed, torch.uint8, "packed", gpu=False)
    _need(scale, torch.float32, "scale", gpu=False)
    if bias is not None:
        _need(bias, torch.float32, "bias", gpu=False)
    if order is not None:
        _need(order, torch.int32, "order", gpu=False)
    if x.dim() != 2 or scale.dim() != 1:
        raise ValueError("x must be [M, K] and scale [N]")
    m, k = x.shape
    n = scale.shape[0]
    if packed.numel() != n * (k // 2):
        raise ValueError("packed must hold N * K / 2 bytes")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    if out is not None:
        _need(out, out_dtype, "out", gpu=False)
    _check_sizes(m, n, k, bias=bias, order=order, out=out)
    _on_gpu(x, packed=packed, scale=scale, bias=bias, order=order, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    need = int(lib.woq_linear_int4_rows_workspace_bytes(m, n, k, int(order is not None)))
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() if (need and workspace is not None) else 0
    _check(lib.woq_linear_int4_rows(_ptr(x), m, _ptr(packed), _ptr(scale), _ptr(bias), _ptr(order), n, k,
                                    F32 if out_dtype == torch.float32 else BF16, _ptr(out),
                                    _ptr(workspace) if need else None, wsb, _stream()), "linear_int4_rows")
    return out

