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


def test_block_ranges_cover_every_block_once():
    for nb, parts in ((1, 4), (7, 3), (100, 16), (5, 64), (4096, 7)):
        rs = bench._block_ranges(nb, parts)
        assert rs[0][0] == 0 and rs[-1][1] == nb
        assert all(a[1] == b[0] for a, b in zip(rs, rs[1:]))
        assert len(rs) <= parts and all(b1 > b0 for b0, b1 in rs)


def test_cpu_baseline_reports_one_core_and_all_cores_legs():
    """The oracle timing runs on a small stand-in for the step's tensors; both
    legs report, and the all-cores leg names the threads it used."""
    from types import SimpleNamespace

    import synth

    B, n, g = 256, 2, 4
    S = 4 * B
    cfg = SimpleNamespace(n_nodes=n, gpus_per_node=g, block=B, slice_len=S, chunk_len=n * S)
    step = SimpleNamespace(c=cfg, bucket_np=synth.small_bf16(n * g * S, (0, 501), 1e-3),
                           w_np=synth.small_bf16(512 * 16, (0, 502), 0.01),
                           g_np=synth.small_bf16(512 * 16, (0, 503), 0.01))
    r = bench.cpu_baseline(step)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["cores"] == len(os.sched_getaffinity(0))
    assert r["one_core"]["cores"] == 1 and r["one_core"]["value"] > 0
    assert set(r["per_kernel_s"]) == set(r["one_core"]["per_kernel_s"]) == {
        "reorder", "quantize_int4_b256", "hop1", "hop2", "quantize_int8_b512", "dequantize_int8_b512",
        "quantize_int4_b128"}
