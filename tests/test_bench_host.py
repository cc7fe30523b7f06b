"""Host-side logic of bench.py (no GPU needed)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_traffic_record_needs_matching_kernel_sources(tmp_path, monkeypatch):
    key = "dequantize_int8_b512_gqa_weight"
    current = bench.source_hash("dequantize")
    recs = {key: {"bytes_per_launch": 123456, "source_hash": current},
            "stale_row": {"bytes_per_launch": 7, "source_hash": "0" * 16}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(recs))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda family: current)
    assert bench.traffic_record(key, "dequantize") == 123456
    assert bench.traffic_record("stale_row", "dequantize") is None
    assert bench.traffic_record("no_such_row", "dequantize") is None


def test_every_row_names_a_known_kernel_family():
    assert set(bench.KERNEL_SOURCES) == {"quantize", "dequantize", "reorder", "drr"}
    for fam, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "block_quantization_codec_amd", "csrc", f)), (fam, f)
