"""Shared helpers of the GPU parity tests (no arithmetic of the method here)."""
import numpy as np
import torch

# Gate on the linear layer's output (max relative error 2e-3 against the
# float64 oracle), read normwise: max|y - y_ref| / max|y_ref| per call.
REL_TOL = 2e-3
# The float32 path sums exact products in float32 (per group, then scaled), so
# its normwise error is a few float32 units times a modest growth factor; a
# much larger error means a wrong term even when it is below the gate.
F32_PATH_TOL = 1e-4
BF16_UNIT = 2.0 ** -8


def to_dev_bf16(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def check_linear(y: torch.Tensor, y_ref: np.ndarray, what: str):
    """Apply the parity gate to a float32 or bfloat16 GPU result."""
    if y.dtype == torch.float32:
        yv = y.detach().cpu().numpy().astype(np.float64)
    else:
        yv = bf16_tensor_to_f64(y)
    assert yv.shape == y_ref.shape, (what, yv.shape, y_ref.shape)
    assert np.all(np.isfinite(yv)), f"{what}: non-finite output"
    scale = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    err = np.abs(yv - y_ref)
    if y.dtype == torch.float32:
        rel = float(np.max(err)) / scale if scale > 0 else float(np.max(err))
        assert rel <= REL_TOL, f"{what}: normwise relative error {rel:.3e} > {REL_TOL}"
        assert rel <= F32_PATH_TOL, f"{what}: float32-path error {rel:.3e} > {F32_PATH_TOL}"
        return rel
    bound = REL_TOL * scale + BF16_UNIT * np.abs(y_ref)
    worst = float(np.max(err - bound)) if err.size else -1.0
    assert worst <= 0, f"{what}: bf16 output outside 2e-3*max|y| + 2^-8*|y| by {worst:.3e}"
    return float(np.max(err)) / scale if scale > 0 else 0.0
