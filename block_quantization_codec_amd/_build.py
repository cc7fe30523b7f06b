"""Build ``libzpp.so`` (the HIP codec library) for gfx950 with hipcc, in-tree.

Usage: ``python block_quantization_codec_amd/_build.py`` (by path: importing
the package needs the library this builds). Objects go to
``_build/`` at the repository root; the library is written next to this file.
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
LIB = os.path.join(PKG, "libzpp.so")
OBJDIR = os.path.join(ROOT, "_build", "zpp")
ARCH = os.environ.get("ZPP_OFFLOAD_ARCH", "gfx950")

DRR_UNITS = [f"drr_in{i}_out{o}.hip" for i in (4, 8) for o in (0, 4, 8)]
SOURCES = ["quantize.hip", "dequantize.hip", "reorder.hip", "drr.hip", *DRR_UNITS, "zpp_api.hip"]
HEADERS = ["zpp_device.h", "zpp_launch.h", "drr_kernel.h"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # binary32 semantics: no contraction into FMA, IEEE division, denormals kept
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the codec library needs the ROCm toolchain to build")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every source and link ``libzpp.so``. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    # the hop-kernel units take longest: start them first
    order = sorted(SOURCES, key=lambda f: not f.startswith("drr_in"))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, order))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    """True when the library is missing or older than any of its sources."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    inc = os.path.join(ROOT, "include", "zpp.h")
    return any(os.path.getmtime(os.path.join(CSRC, f)) > t for f in SOURCES + HEADERS) or \
        os.path.getmtime(inc) > t


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
