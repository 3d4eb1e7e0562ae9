import os
import sys
from fractions import Fraction
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (seconds to minutes)")


def load_golden(name):
    """Parse a ``key: value`` fixture file (lines starting with '#' are citations)."""
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(":")
        out[key.strip()] = val.strip()
    return out


def parse_nums(text):
    vals = []
    for tok in text.split():
        vals.append(Fraction(tok))
    return vals


@pytest.fixture(scope="session")
def gpu_available():
    try:
        import torch
    except Exception:
        return False
    return bool(torch.cuda.is_available())


@pytest.fixture(scope="session")
def woq(gpu_available):
    """The HIP library's Python binding; GPU tests skip only when no GPU exists.

    On a GPU host a missing or broken library is an error, never a skip.
    """
    if not gpu_available:
        pytest.skip("no GPU on this host")
    import weight_only_quantization_amd as w
    w.load()            # raises if libwoq.so is missing or fails to load
    return w
