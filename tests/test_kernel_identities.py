"""Host checks of the arithmetic identities the GPU kernels use in place of
slower operations (the kernels' results are separately compared with the
oracle on the GPU). Quick sampled sweeps by default; set
ZPP_EXHAUSTIVE_IDENTITIES=1 for the exhaustive ones (several minutes):
every significand of five binades for the block-scale identity, every
(x, absmax) pair of finite bfloat16 values for Markstein's division,
about 3.6e9 near-tie binary32 values, and every significand of twelve
binades (subnormal ones included) for the 4- and 8-bit product shortcuts.
"""
from __future__ import annotations

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host_checks", "codec_identities.c")
FULL = os.environ.get("ZPP_EXHAUSTIVE_IDENTITIES") == "1"


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("ident") / "codec_identities")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-msse2", "-mfpmath=sse",
                    "-o", out, SRC, "-lm"], check=True)
    return out


def _run(exe, mode, param):
    r = subprocess.run([exe, mode, str(param)], capture_output=True, text=True, timeout=3600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


def test_block_scale_identity(exe):
    _run(exe, "scale", 5 if FULL else 1)


def test_markstein_codes_on_bf16_domain(exe):
    _run(exe, "markstein", 1 if FULL else 61)


def test_markstein_quotients_near_ties(exe):
    _run(exe, "ties", 2_000_000 if FULL else 3_000)


def test_nibble_products_by_fused_multiply_add(exe):
    _run(exe, "nibble", 1 if FULL else 997)


def test_byte_products_by_fused_multiply_add(exe):
    _run(exe, "byte", 8 if FULL else 4099)
