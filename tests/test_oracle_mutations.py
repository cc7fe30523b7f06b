"""Planted mistakes in the oracle must fail its pins.

Each case below plants one plausible slip in a scratch copy of the C oracle
(``oracle/zpp_oracle.c``): a wrong Q, the nibble order, the rounding rule, a
fused multiply-add or a reversed order in the hop sum, a transposed reorder,
a reciprocal in place of a division, a missing absolute value, bf16
truncation or ties away from zero, a bf16 decode one bit off, unsigned
nibbles, a missing negative clamp, the inverse scale stored, a hop sum
started from -0, an average over the wrong count. The copy is
built and the oracle's pin tests run against it, in a process of their own;
every mutant must make at least one of them fail. This checks the pins, not
the oracle: it shows that none of these mistakes could hide in the oracle
behind tests that pass. Host-side only (gcc and the CPU).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["test_oracle_pins.py", "test_average_oracle.py", "test_twohop_oracle.py",
             "test_oracle_numpy_crosscheck.py"]

# (name, exact text in zpp_oracle.c, replacement)
MUTANTS = [
    ("Q of 8-bit codes off by one", "return bits == 8 ? 127 : 7;", "return bits == 8 ? 126 : 7;"),
    ("Q of 4-bit codes off by one", "return bits == 8 ? 127 : 7;", "return bits == 8 ? 127 : 8;"),
    ("scale through a reciprocal", "float s = a / (float)Q;", "float s = a * (1.0f / (float)Q);"),
    ("absmax without abs", "float m = fabsf(x[i]);", "float m = x[i];"),
    ("quotient through a reciprocal", "float t = x[i] / s;", "float t = x[i] * (1.0f / s);"),
    ("ties away from zero", "float r = rintf(t);", "float r = roundf(t);"),
    ("truncation instead of rounding", "float r = rintf(t);", "float r = truncf(t);"),
    ("no clamp to [-Q, Q]", "if (r > (float)Q)\n                r = (float)Q;", "if (0)\n                r = (float)Q;"),
    ("nibble order swapped on store", "if (i & 1)\n        *byte", "if (!(i & 1))\n        *byte"),
    ("nibbles read as unsigned", "return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    ("bf16 output truncated", "u += 0x7fffu + keep_lsb;", "u += 0u * keep_lsb;"),
    ("reorder transposed", "int64_t owner = node * gpus_per_node + local;",
     "int64_t owner = local * n_nodes + node;"),
    ("hop sum in reverse input order", "for (int32_t r = 0; r < n_inputs; ++r) {",
     "for (int32_t r = n_inputs - 1; r >= 0; --r) {"),
    ("product fused into the hop sum",
     "float v = (float)code_load(c, bits, i) * s[i / block];\n            acc = acc + v;",
     "acc = fmaf((float)code_load(c, bits, i), s[i / block], acc);"),
    ("hop sum averaged over its inputs", "sum[i] = acc;", "sum[i] = acc / (float)n_inputs;"),
    ("average over the input count", "const float d = (float)divisor;", "const float d = (float)n_inputs;"),
    ("hop sum started from -0", "float acc = 0.0f;", "float acc = -0.0f;"),
    ("negative quotients not clamped", "if (r < (float)-Q)\n                r = (float)-Q;",
     "if (0)\n                r = (float)-Q;"),
    ("bf16 decoded one bit low", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("bf16 ties rounded away from zero", "u += 0x7fffu + keep_lsb;", "u += 0x8000u + 0u * keep_lsb;"),
    ("inverse scale stored", "*scale_out = s;", "*scale_out = 1.0f / s;"),
]


def _run_mutant(base: str, idx: int, old: str | None, new: str | None) -> tuple[int, str]:
    d = os.path.join(base, f"m{idx}")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(d, "synth"), ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(d, "tests"))
    for f in ["conftest.py", "twohop_sim.py", *PIN_TESTS]:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    src = os.path.join(d, "oracle", "zpp_oracle.c")
    if old is not None:  # None: the unmodified copy (the control run)
        text = open(src).read()
        assert text.count(old) == 1, f"mutation target not found exactly once: {old!r}"
        open(src, "w").write(text.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join("tests", f) for f in PIN_TESTS]],
                       cwd=d, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-600:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    jobs = [(i, old, new) for i, (_, old, new) in enumerate(MUTANTS)] + [(len(MUTANTS), None, None)]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda a: _run_mutant(str(tmp_path), *a), jobs))
    control_rc, control_out = results.pop()
    assert control_rc == 0, f"the unmodified copy must pass its pins:\n{control_out}"
    survivors = [name for (name, _, _), (rc, _) in zip(MUTANTS, results) if rc == 0]
    broken = [(name, out) for (name, _, _), (rc, out) in zip(MUTANTS, results) if rc not in (0, 1)]
    assert not broken, f"mutants that did not run their tests cleanly: {broken}"
    assert not survivors, f"planted mistakes no pin detects: {survivors}"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutation_targets_exist(name, old, new):
    """Each planted mistake edits text the oracle really contains (once)."""
    text = open(os.path.join(ROOT, "oracle", "zpp_oracle.c")).read()
    assert text.count(old) == 1, name
