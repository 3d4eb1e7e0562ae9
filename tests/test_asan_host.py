"""The C ABI's host-side validation under AddressSanitizer (CPU only).

Every library source is compiled with the sanitizer on its host code only
(the device code is built as usual), linked into a separate copy of the
library, and driven by a small C program (tests/native/abi_validation.c)
that makes every kind of call the library must refuse before touching a GPU:
bad shapes, NULL and misaligned pointers, short workspaces, bad grouped-call
tables, every plan and workspace size class with plan buffers from 1 byte up.
The program checks each status; the sanitizer aborts on any out-of-bounds or
use-after-free access in the host code.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

from weight_only_quantization_amd import _build

ROOT = Path(__file__).resolve().parents[1]
DRIVER = Path(__file__).resolve().parent / "native" / "abi_validation.c"
CLANG = Path("/opt/rocm/llvm/bin/clang")


def test_abi_validation_under_asan(tmp_path):
    hipcc = _build.hipcc()
    if not Path(hipcc).exists() or not CLANG.exists():
        pytest.skip("hipcc or the ROCm clang is not installed")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = tmp_path / (Path(src).stem + ".o")
        proc = subprocess.run([hipcc, *_build.COMMON_FLAGS, *host_asan, "-c", str(_build.CSRC / src), "-o", str(obj)],
                              capture_output=True, text=True)
        return obj, proc

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, _build.SOURCES))
    for (obj, proc), src in zip(results, _build.SOURCES):
        assert proc.returncode == 0, f"{src}: {proc.stderr[-2000:]}"
    lib = tmp_path / "libwoq_asan.so"
    proc = subprocess.run([hipcc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", "-o", str(lib),
                           *[str(o) for o, _ in results]], capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    exe = tmp_path / "abi_validation"
    proc = subprocess.run([str(CLANG), "-fsanitize=address", "-fno-omit-frame-pointer", "-g",
                           f"-I{ROOT / 'include'}", str(DRIVER), f"-L{tmp_path}", "-lwoq_asan",
                           f"-Wl,-rpath,{tmp_path}", "-o", str(exe)], capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "all checks passed" in run.stdout
