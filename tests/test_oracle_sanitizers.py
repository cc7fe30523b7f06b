"""The C oracle under the host compiler's sanitizers.

A scratch copy of the oracle is built with gcc's UndefinedBehaviorSanitizer
(any report aborts) or AddressSanitizer (the Python process preloads its
runtime), and the oracle's pin tests run against it in a process of their
own. Host code only: nothing here touches a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["test_oracle_pins.py", "test_average_oracle.py", "test_twohop_oracle.py",
             "test_oracle_numpy_crosscheck.py"]
BASE_FLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-mfpmath=sse", "-msse2", "-fPIC",
              "-shared", "-fno-omit-frame-pointer"]


def _runtime(name: str) -> str | None:
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.parametrize("kind", ["undefined", "address"])
def test_oracle_pins_pass_under_sanitizer(tmp_path, kind):
    runtime = _runtime("libubsan.so" if kind == "undefined" else "libasan.so")
    if runtime is None:
        pytest.skip(f"gcc has no {kind} sanitizer runtime here")
    d = tmp_path / "copy"
    shutil.copytree(os.path.join(ROOT, "oracle"), d / "oracle", ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), d / "synth", ignore=shutil.ignore_patterns("__pycache__"))
    (d / "tests").mkdir()
    for f in ["conftest.py", "twohop_sim.py", *PIN_TESTS]:
        shutil.copy(os.path.join(ROOT, "tests", f), d / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), d / "tests" / "golden")
    so = d / "oracle" / "liboracle.so"
    flags = [f"-fsanitize={kind}"] + (["-fno-sanitize-recover=undefined"] if kind == "undefined" else [])
    subprocess.run(["gcc", *BASE_FLAGS, *flags, "-o", str(so), str(d / "oracle" / "zpp_oracle.c"), "-lm"],
                   check=True)
    later = os.path.getmtime(d / "oracle" / "zpp_oracle.c") + 3600
    os.utime(so, (later, later))  # newer than the source: the oracle loads it as built
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    if kind == "address":
        env["LD_PRELOAD"] = runtime
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join("tests", f) for f in PIN_TESTS]],
                       cwd=d, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
