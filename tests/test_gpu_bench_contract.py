"""bench.py's one JSON line, from a short run on the GPU.

Runs ``bench.py --steps 2 --warmup 1 --no-cpu-baseline`` in a process of its
own and checks the line's contract: the fields and their types, one GPU,
the step counts asked for, the roofline object (its fraction is achieved over
peak, against the 8 TB/s HBM peak) and the measured copy ceiling each row is
compared with. The CPU-baseline leg is skipped here (it only times the oracle).
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    need_gpu()
    print("running bench.py --steps 2 --warmup 1 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])

    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["data"] == "synthetic" and d["vs_baseline"] is None and d["dtype"] == "f32"
    assert isinstance(d["metric"], str) and d["metric"]
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert isinstance(d["config"]["workload"], str) and d["config"]["workload"]
    assert d["cpu_baseline"] is None

    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    rows = d["kernels"]
    assert rf["kernel"] in rows
    assert rows[rf["kernel"]]["ms"] == max(v["ms"] for v in rows.values())

    assert d["graph_step"]["ms_per_step"] > 0 and d["graph_step"]["value"] > 0

    cp = d["copy_ceiling"]
    assert cp["bytes"] == 2 << 30 and cp["GBps"] > 0
    for name, v in rows.items():
        assert v["ms"] > 0 and 0 < v["hbm_frac"] < 1, name
        assert abs(v["copy_frac"] - v["rw_GBps"] / cp["GBps"]) < 2e-3, name
