"""Build the C client of the codec (``zpp_client``) with the host C compiler.

It includes ``include/zpp.h``, links ``libzpp.so`` and the HIP runtime, and
finds the library at run time relative to its own location.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "zpp_client.c")
BIN = os.path.join(HERE, "zpp_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", BIN,
           "-L", os.path.join(ROOT, "block_quantization_codec_amd"), "-lzpp",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../block_quantization_codec_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    print(build())
