"""The library's host code (argument validation, the C ABI) under clang's sanitizers.

``zpp_api.hip`` is compiled with UndefinedBehaviorSanitizer or
AddressSanitizer on its host side only (``-Xarch_host``; device code is
built as usual), linked with the kernel objects ``build()`` left in
``_build/zpp``, and the ABI tests run against that library in a process of
their own with the sanitizer runtime preloaded. No GPU is used: every ABI test
fails in the host-side checks before any HIP call that needs a device.
"""
from __future__ import annotations

import glob
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_quantization_codec_amd")
OBJDIR = os.path.join(ROOT, "_build", "zpp")
RUNTIMES = {"undefined": "libclang_rt.ubsan_standalone-x86_64.so", "address": "libclang_rt.asan-x86_64.so"}


def _build_module():
    spec = importlib.util.spec_from_file_location("zpp_build_for_sanitizers", os.path.join(PKG, "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("kind", ["undefined", "address"])
def test_abi_tests_pass_under_host_sanitizer(tmp_path, kind):
    b = _build_module()
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc here")
    runtime = sorted(glob.glob(f"/opt/rocm/llvm/lib/clang/*/lib/linux/{RUNTIMES[kind]}"))
    kernel_objs = [os.path.join(OBJDIR, os.path.splitext(f)[0] + ".o") for f in b.SOURCES if f != "zpp_api.hip"]
    if not runtime:
        pytest.skip(f"no clang {kind} sanitizer runtime here")
    if not all(os.path.exists(o) for o in kernel_objs):
        pytest.skip("kernel objects missing: run __graft_entry__.build() first")

    d = tmp_path / "copy"
    shutil.copytree(PKG, d / "block_quantization_codec_amd", ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    for sub in ("include", "oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), d / sub, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    (d / "tests").mkdir()
    for f in ("conftest.py", "test_abi.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), d / "tests" / f)

    san = ["-Xarch_host", f"-fsanitize={kind}"]
    if kind == "undefined":
        san += ["-Xarch_host", "-fno-sanitize-recover=undefined"]
    api_obj = str(tmp_path / "zpp_api.o")
    flags = [f if f != "-O3" else "-O1" for f in b.HIPCC_FLAGS]
    subprocess.run([hipcc, *flags, "-g", *san, "-c", os.path.join(PKG, "csrc", "zpp_api.hip"), "-o", api_obj],
                   check=True, capture_output=True)
    link = [hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-Xarch_host", f"-fsanitize={kind}"]
    if kind == "address":
        link += ["-shared-libasan"]
    subprocess.run([*link, "-o", str(d / "block_quantization_codec_amd" / "libzpp.so"), *kernel_objs, api_obj],
                   check=True, capture_output=True)

    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", LD_PRELOAD=runtime[-1],
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join("tests", "test_abi.py")], cwd=d, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
