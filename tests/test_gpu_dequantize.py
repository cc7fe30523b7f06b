"""GPU parity of zpp_dequantize_blocks against the CPU oracle.

The expected value is the binary32 product code * scale (bf16 output: that
product rounded to nearest-even), so parity is checked bit for bit; the
codec's stated tolerance (1e-5 of the block scale) is asserted as well.
Inputs: arbitrary code bytes (including -128 and -8, which the quantizer
never writes) with scales spanning subnormal to large binades, plus the
hand-derived golden cases and a round trip of quantized workload data.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, assert_bits_equal, assert_within_scale, dev, need_gpu, torch

pytestmark = pytest.mark.gpu

BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _zpp():
    import block_quantization_codec_amd as z
    return z


def _run(codes_np, scales_np, bits, numel, block, out):
    z = _zpp()
    codes = dev(codes_np)
    scales = dev(scales_np)
    isz = 2 if out == "bf16" else 4
    gy = Guarded(numel * isz)
    torch.cuda.synchronize()
    z.zpp_dequantize_blocks(codes, scales, bits, numel, block, gy.ptr,
                            z.ZPP_BF16 if out == "bf16" else z.ZPP_FP32)
    torch.cuda.synchronize()
    assert gy.untouched(), "write outside the output buffer"
    return gy.as_np(np.uint16 if out == "bf16" else np.float32)


def _random_case(numel, block, bits, seed):
    rng = np.random.default_rng([seed, numel, block, bits])
    codes = rng.integers(0, 256, numel * bits // 8, dtype=np.uint8)
    nb = numel // block
    scales = np.exp2(rng.uniform(-140, 100, nb)).astype(np.float32)
    scales[rng.random(nb) < 0.05] = 0.0
    return codes, scales


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("block", BLOCKS)
def test_dequantize_matches_oracle(block, bits, out):
    nb = max(3, 45_000 // block) + 1
    n = nb * block
    codes, scales = _random_case(n, block, bits, 1)
    got = _run(codes, scales, bits, n, block, out)
    want = oracle.dequantize(codes, scales, bits, n, block, out=out)
    assert_bits_equal(got, want, f"dequant B={block} bits={bits} {out}")
    if out == "f32":
        assert_within_scale(got, want, np.repeat(scales, block), "dequant tolerance")


def test_golden_dequantize_on_gpu():
    with open(os.path.join(os.path.dirname(__file__), "golden", "dequantize_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        codes = np.frombuffer(bytes.fromhex(c["codes_hex"]), np.uint8)
        if "scales_bits_hex" in c:
            scales = np.array([int(h, 16) for h in c["scales_bits_hex"]], np.uint32).view(np.float32)
        else:
            scales = np.asarray(c["scales"], np.float32)
        B, bits = c["block"], c["bits"]
        n_real = codes.size * 8 // bits
        # pad each golden block of B to a block of 32 (extra codes are 0)
        per = B * bits // 8
        nb = n_real // B
        padded = np.zeros(nb * 32 * bits // 8, np.uint8)
        for b in range(nb):
            padded[b * 32 * bits // 8:][:per] = codes[b * per:(b + 1) * per]
        for out, key in (("f32", "y_f32"), ("bf16", "y_bf16_hex")):
            if key not in c:
                continue
            y = _run(padded, scales, bits, nb * 32, 32, out).reshape(nb, 32)[:, :B].reshape(-1)
            if out == "f32":
                assert y.tolist() == c[key], c["name"]
            else:
                assert [f"{v:04x}" for v in y.tolist()] == c[key], c["name"]


@pytest.mark.parametrize("bits,block", [(8, 256), (8, 512), (4, 128), (8, 2048)])
def test_round_trip_of_workload_data(bits, block):
    x = synth.small_bf16(block * 500, (5, bits, block), 0.02, 1e-3, 50.0)
    codes, scales = oracle.quantize(x, block, bits)
    got = _run(codes, scales, bits, x.size, block, "bf16")
    assert_bits_equal(got, oracle.dequantize(codes, scales, bits, x.size, block, out="bf16"), "round trip")
    # and the quantizer's error bound holds on what the GPU rebuilt (f32 path)
    y = _run(codes, scales, bits, x.size, block, "f32").astype(np.float64)
    xv = oracle.bf16_decode(x).astype(np.float64)
    assert np.all(np.abs(y - xv) <= np.repeat(scales.astype(np.float64), block) * (0.5 + 2.0 ** -15))


def test_bf16_rounding_of_every_pattern_class():
    """Products landing exactly on bf16 ties, on subnormals, and near overflow."""
    rng = np.random.default_rng(9)
    block = 32
    nb = 4096
    # scales whose low 16 bits are exactly the half-way pattern make code 1 a tie
    sb = (rng.integers(1, 0x7F7F, nb).astype(np.uint32) << 16) | 0x8000
    sb[:256] = rng.integers(1, 0x00800000, 256).astype(np.uint32)  # subnormal scales
    scales = sb.view(np.float32)
    codes = rng.integers(0, 256, nb * block, dtype=np.uint8)
    codes[::block] = 1
    got = _run(codes, scales, 8, nb * block, block, "bf16")
    assert_bits_equal(got, oracle.dequantize(codes, scales, 8, nb * block, block, out="bf16"), "bf16 ties")


def test_empty_is_a_no_op():
    z = _zpp()
    z.zpp_dequantize_blocks(None, None, 8, 0, 256, None, z.ZPP_BF16)
