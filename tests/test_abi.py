"""The C-ABI library on the host: it loads, exports every entry point that
include/zpp.h declares, and rejects invalid arguments before any GPU work.

No kernel is launched here (these run on machines without a GPU): every
argument case below fails in the library's pure host-side checks, which run
before it makes any HIP call.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zpp.h")


def _build_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "zpp_build", os.path.join(ROOT, "block_quantization_codec_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def z():
    b = _build_module()
    if b.stale():
        b.build()
    import block_quantization_codec_amd as z

    return z


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zpp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_codec_calls():
    names = declared_functions()
    for n in ("zpp_quantize_blocks", "zpp_quantize_reordered", "zpp_dequantize_blocks", "zpp_reorder_slices",
              "zpp_dequant_reduce_requant", "zpp_dequant_reduce_average"):
        assert n in names


def test_library_exports_every_declared_symbol(z):
    lib = ctypes.CDLL(z.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", z.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (zpp_[a-z0-9_]+)$", out, flags=re.M))
    assert exported == set(declared_functions())
    assert set(z.EXPORTED) == exported


def test_abi_version_and_status_strings(z):
    assert z.zpp_abi_version() == 2
    for s in range(0, 8):
        assert z.zpp_status_string(s).startswith("ZPP_")
    for bad in (99, -1, 8, -(1 << 31), (1 << 31) - 1):
        assert z.zpp_status_string(bad) == "unknown zpp_status"


def test_pointer_check_switch_returns_the_previous_setting(z):
    """zpp_set_pointer_checks touches no GPU: it only swaps the setting."""
    f = z.library().zpp_set_pointer_checks
    assert f(0) == 1
    assert f(7) == 0          # any non-zero value switches them on
    assert f(1) == 1
    assert z.zpp_set_pointer_checks(True) is True


def test_status_values_match_the_header(z):
    """The numeric status codes: 0-5 as the boundary contract fixes them
    (OK, NULL, ARG, ALIGN, UNSUPPORTED, LAUNCH), the two extra argument
    errors after them; the binding, the header and the library agree."""
    want = {"ZPP_OK": 0, "ZPP_ERR_NULL": 1, "ZPP_ERR_ARG": 2, "ZPP_ERR_ALIGN": 3, "ZPP_ERR_UNSUPPORTED": 4,
            "ZPP_ERR_LAUNCH": 5, "ZPP_ERR_OVERLAP": 6, "ZPP_ERR_POINTER": 7}
    hdr = open(HEADER).read()
    for name, v in want.items():
        assert getattr(z, name) == v, name
        assert re.search(rf"\b{name} = {v}\b", hdr), name
        assert z.zpp_status_string(v).startswith(name), (name, z.zpp_status_string(v))


# Fake device addresses: never dereferenced, because each case fails in the
# pure argument checks that precede every HIP call.
A = 1 << 40  # 16-byte aligned


def test_quantize_argument_errors(z):
    L = z.library()
    q = L.zpp_quantize_blocks
    assert q(A, 3, 256, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG          # dtype
    for bad in (0, -1, -(1 << 31), (1 << 31) - 1):
        assert q(A, bad, 256, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG
    assert q(A, 1, 256, 256, 6, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG          # bits
    assert q(A, 1, 256, 100, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG          # block not pow2
    assert q(A, 1, 256, 16, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG           # block < 32
    assert q(A, 1, 16384, 8192, 8, A + 65536, A + 131072, None) == z.ZPP_ERR_ARG    # block > 4096
    assert q(A, 1, 300, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG          # numel % block
    assert q(A, 1, -256, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG         # negative
    assert q(None, 1, 256, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_NULL
    assert q(A, 1, 256, 256, 8, None, A + 8192, None) == z.ZPP_ERR_NULL
    assert q(A + 2, 1, 256, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ALIGN
    assert q(A, 1, 256, 256, 8, A + 4100, A + 8192, None) == z.ZPP_ERR_ALIGN
    assert q(A, 1, 256, 256, 8, A + 4096, A + 8194, None) == z.ZPP_ERR_ALIGN
    assert q(A, 1, 256, 256, 8, A + 256, A + 8192, None) == z.ZPP_ERR_OVERLAP       # codes in x
    assert q(A, 1, 256, 256, 8, A + 4096, A + 4096 + 128, None) == z.ZPP_ERR_OVERLAP  # scales in codes
    assert q(None, 1, 0, 256, 8, None, None, None) == z.ZPP_OK                        # empty


def test_quantize_reordered_argument_errors(z):
    q = z.library().zpp_quantize_reordered
    S, O = 1 << 12, A + (1 << 30)

    def call(x=A, dt=1, s=S, n=2, g=4, first=0, count=8, block=256, bits=4, codes=O, scales=O + (1 << 20)):
        return q(x, dt, s, n, g, first, count, block, bits, codes, scales, None)

    assert call(dt=5) == z.ZPP_ERR_ARG
    assert call(bits=2) == z.ZPP_ERR_ARG
    assert call(n=0) == z.ZPP_ERR_ARG
    assert call(n=256, g=256) == z.ZPP_ERR_ARG                      # more than 65535 slices
    assert call(s=S + 128) == z.ZPP_ERR_ARG                          # slice not whole blocks
    assert call(block=48) == z.ZPP_ERR_ARG
    assert call(first=-1) == z.ZPP_ERR_ARG
    assert call(first=7, count=2) == z.ZPP_ERR_ARG                  # past the last slice
    assert call(count=-1) == z.ZPP_ERR_ARG
    assert call(x=None) == z.ZPP_ERR_NULL
    assert call(scales=None) == z.ZPP_ERR_NULL
    assert call(x=A + 8) == z.ZPP_ERR_ALIGN
    assert call(codes=O + 4) == z.ZPP_ERR_ALIGN
    assert call(codes=A + 64) == z.ZPP_ERR_OVERLAP                  # codes inside x
    assert call(scales=O + 64) == z.ZPP_ERR_OVERLAP                 # scales inside codes
    assert call(x=None, count=0) == z.ZPP_OK                        # nothing to do
    assert call(x=None, s=0) == z.ZPP_OK


def test_dequantize_argument_errors(z):
    d = z.library().zpp_dequantize_blocks
    assert d(A, A + 4096, 8, 256, 256, A + 8192, 0, None) == z.ZPP_ERR_ARG          # dtype
    for bad in (-1, 3, -(1 << 31), (1 << 31) - 1):
        assert d(A, A + 4096, 8, 256, 256, A + 8192, bad, None) == z.ZPP_ERR_ARG
    assert d(A, A + 4096, 5, 256, 256, A + 8192, 1, None) == z.ZPP_ERR_ARG          # bits
    assert d(A, A + 4096, 8, 257, 256, A + 8192, 1, None) == z.ZPP_ERR_ARG
    assert d(A, None, 8, 256, 256, A + 8192, 1, None) == z.ZPP_ERR_NULL
    assert d(A + 8, A + 4096, 8, 256, 256, A + 8192, 1, None) == z.ZPP_ERR_ALIGN
    assert d(A, A + 4098, 8, 256, 256, A + 8192, 1, None) == z.ZPP_ERR_ALIGN
    assert d(A, A + 4096, 8, 256, 256, A + 64, 1, None) == z.ZPP_ERR_OVERLAP         # y over codes
    assert d(None, None, 8, 0, 256, None, 1, None) == z.ZPP_OK


def test_reorder_argument_errors(z):
    r = z.library().zpp_reorder_slices
    assert r(A, A + (1 << 20), 100, 0, 4, None) == z.ZPP_ERR_ARG
    assert r(A, A + (1 << 20), 100, 2, 0, None) == z.ZPP_ERR_ARG
    assert r(A, A + (1 << 20), -1, 2, 4, None) == z.ZPP_ERR_ARG
    assert r(A, A + (1 << 20), 100, 256, 256, None) == z.ZPP_ERR_ARG                 # > 65535 slices
    assert r(None, A, 100, 2, 4, None) == z.ZPP_ERR_NULL
    assert r(A, A + 400, 100, 2, 4, None) == z.ZPP_ERR_OVERLAP
    assert r(None, None, 0, 2, 4, None) == z.ZPP_OK


def test_drr_argument_errors(z):
    f = z.library().zpp_dequant_reduce_requant
    C, S, O, OS, U = A, A + (1 << 24), A + (1 << 25), A + (1 << 26), A + (1 << 27)
    ok = dict(ci=C, cs=1 << 16, si=S, ss=1 << 10, R=4, bi=4, n=1 << 12, B=256, co=O, so=OS, bo=4, su=U)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["ci"], a["cs"], a["si"], a["ss"], a["R"], a["bi"], a["n"], a["B"], a["co"], a["so"],
                 a["bo"], a["su"], None)

    assert call(bi=2) == z.ZPP_ERR_ARG
    assert call(bo=2) == z.ZPP_ERR_ARG
    assert call(R=0) == z.ZPP_ERR_ARG
    assert call(R=5000) == z.ZPP_ERR_ARG
    assert call(n=300) == z.ZPP_ERR_ARG
    assert call(cs=-16) == z.ZPP_ERR_ARG
    assert call(bo=0, co=None, so=None, su=None) == z.ZPP_ERR_ARG                    # no output
    assert call(bo=0) == z.ZPP_ERR_ARG                                                 # codes_out without bits
    assert call(ci=None) == z.ZPP_ERR_NULL
    assert call(so=None) == z.ZPP_ERR_NULL
    assert call(cs=8) == z.ZPP_ERR_ALIGN
    assert call(ci=C + 4) == z.ZPP_ERR_ALIGN
    assert call(su=U + 4) == z.ZPP_ERR_ALIGN
    assert call(co=C + 64) == z.ZPP_ERR_OVERLAP                                        # output in input
    assert call(so=O + 16) == z.ZPP_ERR_OVERLAP                                        # outputs overlap
    assert call(n=0) == z.ZPP_OK


def test_drr_split_argument_errors(z):
    f = z.library().zpp_dequant_reduce_requant_split
    C, S, O, OS, K, KS = A, A + (1 << 24), A + (1 << 25), A + (1 << 26), A + (1 << 27), A + (1 << 28)
    ok = dict(ci=C, cs=1 << 16, si=S, ss=1 << 10, R=8, bi=4, n=1 << 12, B=256, kb=1024, kl=512, co=O, so=OS,
              kc=K, ks=KS, bo=4)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["ci"], a["cs"], a["si"], a["ss"], a["R"], a["bi"], a["n"], a["B"], a["kb"], a["kl"], a["co"],
                 a["so"], a["kc"], a["ks"], a["bo"], None)

    assert call(bi=2) == z.ZPP_ERR_ARG
    assert call(bo=0) == z.ZPP_ERR_ARG                       # the split step always requantizes
    assert call(bo=16) == z.ZPP_ERR_ARG
    assert call(R=0) == z.ZPP_ERR_ARG
    assert call(n=300) == z.ZPP_ERR_ARG
    assert call(B=48) == z.ZPP_ERR_ARG
    assert call(kb=-256) == z.ZPP_ERR_ARG
    assert call(kl=-256) == z.ZPP_ERR_ARG
    assert call(kb=128) == z.ZPP_ERR_ARG                     # window not whole blocks
    assert call(kl=100) == z.ZPP_ERR_ARG
    assert call(kb=4096, kl=256) == z.ZPP_ERR_ARG            # window past the end
    assert call(kb=1 << 62, kl=1 << 62) == z.ZPP_ERR_ARG     # no wrap-around in the end check
    assert call(kb=0, kl=(1 << 12) + 256) == z.ZPP_ERR_ARG
    assert call(ci=None) == z.ZPP_ERR_NULL
    assert call(co=None) == z.ZPP_ERR_NULL                   # elements left to send
    assert call(ks=None) == z.ZPP_ERR_NULL                   # a window to keep
    assert call(cs=8) == z.ZPP_ERR_ALIGN
    assert call(kc=K + 4) == z.ZPP_ERR_ALIGN
    assert call(so=OS + 2) == z.ZPP_ERR_ALIGN
    assert call(kc=C + 64) == z.ZPP_ERR_OVERLAP              # output inside an input
    assert call(ks=O + 16) == z.ZPP_ERR_OVERLAP              # outputs overlap each other
    assert call(kc=OS) == z.ZPP_ERR_OVERLAP
    assert call(n=0) == z.ZPP_ERR_ARG                        # the window no longer fits
    assert call(n=0, kb=0, kl=0) == z.ZPP_OK
    assert call(n=0, kb=0, kl=0, ci=None, co=None, kc=None) == z.ZPP_OK


def test_drr_average_argument_errors(z):
    f = z.library().zpp_dequant_reduce_average
    C, S, U = A, A + (1 << 24), A + (1 << 27)
    ok = dict(ci=C, cs=1 << 16, si=S, ss=1 << 10, R=32, bi=4, n=1 << 12, B=256, d=256, av=U)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["ci"], a["cs"], a["si"], a["ss"], a["R"], a["bi"], a["n"], a["B"], a["d"], a["av"], None)

    assert call(bi=0) == z.ZPP_ERR_ARG
    assert call(R=0) == z.ZPP_ERR_ARG
    assert call(B=100) == z.ZPP_ERR_ARG
    assert call(ss=-1) == z.ZPP_ERR_ARG
    assert call(d=0) == z.ZPP_ERR_ARG
    assert call(d=-3) == z.ZPP_ERR_ARG
    assert call(d=z.ZPP_MAX_DIVISOR + 1) == z.ZPP_ERR_ARG
    assert call(av=None) == z.ZPP_ERR_NULL
    assert call(si=None) == z.ZPP_ERR_NULL
    assert call(av=U + 8) == z.ZPP_ERR_ALIGN
    assert call(cs=24) == z.ZPP_ERR_ALIGN
    assert call(av=C + 256) == z.ZPP_ERR_OVERLAP
    assert call(av=S) == z.ZPP_ERR_OVERLAP
    assert call(n=0) == z.ZPP_OK
    assert call(n=0, av=None) == z.ZPP_OK


def test_sizes_beyond_the_limit_are_refused(z):
    """Element counts, strides and reordered buffers past ZPP_MAX_NUMEL are
    refused before any byte range is computed, so no 64-bit product can wrap
    round to a small or negative size; the limit itself passes (these calls
    then stop at the overlap check, which needs no GPU)."""
    L, M = z.library(), z.ZPP_MAX_NUMEL
    q, d = L.zpp_quantize_blocks, L.zpp_dequantize_blocks
    for n in (M + 256, 1 << 62, (1 << 63) - 256):
        assert q(A, 1, n, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_ARG
        assert d(A, A + 4096, 4, n, 256, A + 8192, 1, None) == z.ZPP_ERR_ARG
    assert q(A, 1, M, 256, 8, A + 4096, A + 8192, None) == z.ZPP_ERR_OVERLAP
    assert d(A, A + 4096, 4, M, 256, A + 8192, 1, None) == z.ZPP_ERR_OVERLAP

    qr = L.zpp_quantize_reordered
    assert qr(A, 1, (M // 8) + 256, 2, 4, 0, 8, 256, 4, A + 64, A + 128, None) == z.ZPP_ERR_ARG
    assert qr(A, 1, 1 << 60, 2, 4, 0, 8, 256, 4, A + 64, A + 128, None) == z.ZPP_ERR_ARG
    assert qr(A, 1, M // 8, 2, 4, 0, 8, 256, 4, A + 64, A + 128, None) == z.ZPP_ERR_OVERLAP

    r = L.zpp_reorder_slices
    assert r(A, A + 64, (4 * M) // 8 + 1, 2, 4, None) == z.ZPP_ERR_ARG
    assert r(A, A + 64, 1 << 61, 2, 4, None) == z.ZPP_ERR_ARG
    assert r(A, A + 64, (4 * M) // 8, 2, 4, None) == z.ZPP_ERR_OVERLAP

    f, g = L.zpp_dequant_reduce_requant, L.zpp_dequant_reduce_average
    C, S, O, OS, U = A, A + (1 << 24), A + (1 << 25), A + (1 << 26), A + (1 << 27)

    def drr(n=1 << 12, cs=1 << 16, ss=1 << 10, co=O):
        return f(C, cs, S, ss, 4, 4, n, 256, co, OS, 4, U, None)

    def avg(n=1 << 12, cs=1 << 16, ss=1 << 10, av=U):
        return g(C, cs, S, ss, 32, 4, n, 256, 256, av, None)

    for call, out in ((drr, "co"), (avg, "av")):
        assert call(n=M + 256) == z.ZPP_ERR_ARG
        assert call(n=1 << 62) == z.ZPP_ERR_ARG
        assert call(cs=M + 16) == z.ZPP_ERR_ARG
        assert call(cs=(1 << 63) - 16) == z.ZPP_ERR_ARG
        assert call(ss=M + 1) == z.ZPP_ERR_ARG
        assert call(ss=1 << 62) == z.ZPP_ERR_ARG
        # at the limits every range stays exact: the output inside the inputs is still seen
        assert call(n=M, cs=M, ss=M, **{out: C + 64}) == z.ZPP_ERR_OVERLAP


def test_helpers_refuse_strided_views(z):
    """The allocating helpers hand data_ptr() to flat-buffer kernels, so a
    strided view is refused before any call (no GPU needed to see it)."""
    import torch

    t = torch.zeros(64, 64).t()
    c = torch.zeros(64, 64, dtype=torch.uint8)[:, ::2]
    s = torch.zeros(8, 8)[:, ::2]
    calls = [lambda: z.quantize(t, 32, 8), lambda: z.quantize_reordered(t, 2, 2, 32, 4),
             lambda: z.dequantize(c, torch.zeros(64), 8, 2048, 32),
             lambda: z.dequantize(torch.zeros(2048, dtype=torch.uint8), s, 8, 1024, 32),
             lambda: z.reorder(t, 2, 2), lambda: z.dequant_reduce_requant(c, torch.zeros(64), 2, 8, 1024, 32),
             lambda: z.dequant_reduce_average(torch.zeros(2048, dtype=torch.uint8), s, 2, 8, 1024, 32, 2)]
    for call in calls:
        with pytest.raises(ValueError, match="contiguous"):
            call()


def test_oracle_and_library_share_no_code():
    """The product sources never mention the oracle, and the oracle never the product."""
    pkg = os.path.join(ROOT, "block_quantization_codec_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), fn
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", fn)).read()
            assert not re.search(r"^\s*(import|from)\s+block_quantization_codec_amd", text, re.M), fn
            assert not re.search(r"#\s*include\s*[<\"].*zpp", text), fn
            assert "libzpp" not in text, fn


def test_import_fails_loudly_without_the_library(tmp_path):
    """The binding has no fallback: a copy of the package with no libzpp.so
    beside it refuses to import, naming the missing library."""
    import shutil
    import sys
    pkg = os.path.join(ROOT, "block_quantization_codec_amd")
    dst = tmp_path / "block_quantization_codec_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    r = subprocess.run([sys.executable, "-c", "import block_quantization_codec_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libzpp.so is missing" in r.stderr
