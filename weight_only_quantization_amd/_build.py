"""Compile libwoq.so for gfx950 with hipcc (in tree, next to this file).

Each HIP source is compiled to an object in parallel, then linked into one
shared library.  Runs on a host without a GPU (hipcc cross-compiles).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libwoq.so"

SOURCES = ["api.hip", "codec.hip", "linear_rows.hip", "linear_gemv.hip", "linear_skinny.hip", "linear_smallm.hip", "linear_gemm.hip", "gptq.hip", "awq.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    # Packed float32 instructions are kept out of all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return path


def _compile(src: str, extra: list[str]) -> tuple[str, int, str]:
    obj = BUILD / (Path(src).stem + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", str(CSRC / src), "-o", str(obj)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    return str(obj), proc.returncode, out


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> Path:
    """Compile every source and link libwoq.so; raises on any compiler error."""
    BUILD.mkdir(exist_ok=True)
    extra = list(extra_flags or [])
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    errors = []
    for (obj, rc, out), src in zip(results, SOURCES):
        if out.strip() and (verbose or rc):
            print(f"[{src}]\n{out}", file=sys.stderr)
        if rc:
            errors.append(src)
    if errors:
        raise RuntimeError(f"hipcc failed for {errors}")
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
           *[r[0] for r in results]]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode:
        raise RuntimeError("link failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
