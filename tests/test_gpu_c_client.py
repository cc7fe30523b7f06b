"""The codec used from plain C: tests/c_client/zpp_client.c.

The client (built by ``__graft_entry__.build()``) allocates with hipMalloc,
calls every entry point through ``include/zpp.h`` (the fused reorder +
quantize and the split hop step included) on a stream of its own and
writes the results to files; this test feeds it a seeded input, runs it as a
child process and compares everything with the oracle bit for bit. It also
checks the client saw ordinary host memory refused with ZPP_ERR_POINTER.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_bits_equal, need_gpu

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c_client", "zpp_client")


def test_c_client_matches_oracle(tmp_path):
    need_gpu()
    if not os.path.exists(CLIENT):
        raise AssertionError(f"{CLIENT} is missing: run __graft_entry__.build() first")
    import block_quantization_codec_amd as z

    B, S = 256, 256 * 37
    n = 8 * S
    x = synth.small_bf16(n, (0, 701), 1e-3, 1e-3, 20.0)
    x.tofile(tmp_path / "x.bin")
    (tmp_path / "params.txt").write_text(f"{n} {S} {B}\n")
    r = subprocess.run([CLIENT, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    def read(name, dtype):
        return np.fromfile(tmp_path / name, dtype=dtype)

    c8, s8 = oracle.quantize(x, B, 8)
    assert_bits_equal(read("codes8.bin", np.uint8), c8, "8-bit codes")
    assert_bits_equal(read("scales8.bin", np.float32), s8, "8-bit scales")
    assert_bits_equal(read("y.bin", np.uint16), oracle.dequantize(c8, s8, 8, n, B, out="bf16"), "bf16 dequantized")
    re = oracle.reorder_slices(x, 2, 4)
    assert_bits_equal(read("reordered.bin", np.uint16), re, "reordered")
    c4, s4 = oracle.quantize(re, B, 4)
    assert_bits_equal(read("codes4.bin", np.uint8), c4, "4-bit codes")
    assert_bits_equal(read("scales4.bin", np.float32), s4, "4-bit scales")
    cl = [c4[k * S // 2:(k + 1) * S // 2] for k in range(8)]
    sl = [s4[k * S // B:(k + 1) * S // B] for k in range(8)]
    co, so, su = oracle.dequant_reduce_requant(cl, sl, 4, S, B, 4)
    assert_bits_equal(read("sum.bin", np.float32), su, "hop sum")
    assert_bits_equal(read("hop_codes.bin", np.uint8), co, "hop codes")
    assert_bits_equal(read("hop_scales.bin", np.float32), so, "hop scales")
    assert_bits_equal(read("avg.bin", np.float32), oracle.dequant_average(cl, sl, 4, S, B, 8), "average")
    assert_bits_equal(read("fused_codes.bin", np.uint8), c4, "fused reorder+quantize codes")
    assert_bits_equal(read("fused_scales.bin", np.float32), s4, "fused reorder+quantize scales")
    k0, k1 = 10 * B, 17 * B  # the split hop's kept window
    assert_bits_equal(read("keep_codes.bin", np.uint8), co[k0 // 2:k1 // 2], "split hop kept codes")
    assert_bits_equal(read("keep_scales.bin", np.float32), so[k0 // B:k1 // B], "split hop kept scales")
    assert_bits_equal(read("send_codes.bin", np.uint8), np.concatenate([co[:k0 // 2], co[k1 // 2:]]),
                      "split hop sent codes")
    assert_bits_equal(read("send_scales.bin", np.float32), np.concatenate([so[:k0 // B], so[k1 // B:]]),
                      "split hop sent scales")
    status = dict(line.split() for line in (tmp_path / "status.txt").read_text().splitlines())
    assert int(status["host_pointer"]) == z.ZPP_ERR_POINTER
    assert int(status["abi"]) == z.zpp_abi_version()
