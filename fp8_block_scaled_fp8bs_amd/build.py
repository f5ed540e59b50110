"""Build libfp8bs.so in-tree with hipcc for gfx950.

The library is plain C ABI (include/fp8bs.h); the Python binding loads it
with ctypes. Translation units are compiled in parallel, then linked.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libfp8bs.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["fp8bs_api.hip"] + sorted(
    f for f in os.listdir(CSRC) if f.startswith("fp8bs_kern_") and f.endswith(".hip"))

ARCH = "gfx950"

# No fast-math: the quantizers need correctly rounded fp32 division and IEEE
# subnormals. Packed fp32 instructions are disabled.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfp8bs")


def _flags_string() -> str:
    return " ".join(f for f in HIP_FLAGS if not f.startswith("-W"))


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}",
           f'-DFP8BS_BUILD_FLAGS="{_flags_string()}"',
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libfp8bs.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
