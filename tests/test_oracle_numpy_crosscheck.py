"""A second, independent host implementation (vectorized NumPy binary32) of
the codec's arithmetic, checked bit for bit against the C oracle.

The two share nothing but the readings: NumPy's float32 division,
multiplication and addition are single IEEE binary32 operations (rounded to
nearest even, never fused) and ``np.rint`` rounds half to even, so both must
produce the same bits. The pins of the readings themselves live in
``test_oracle_pins.py``; this catches slips in either implementation (an
index, a nibble order, a clamp, a summation order).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

QMAX = {8: 127, 4: 7}


def np_decode_bf16(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def np_quantize(x: np.ndarray, block: int, bits: int):
    """Symmetric absmax block quantization in binary32."""
    xf = np_decode_bf16(x) if x.dtype == np.uint16 else x.astype(np.float32)
    xb = xf.reshape(-1, block)
    a = np.abs(xb).max(axis=1)
    s = a / np.float32(QMAX[bits])
    with np.errstate(divide="ignore", invalid="ignore"):
        t = xb / s[:, None]
    q = np.where(s[:, None] == 0, np.float32(0), np.clip(np.rint(t), -QMAX[bits], QMAX[bits])).astype(np.int64)
    q = q.reshape(-1)
    if bits == 8:
        codes = (q & 0xFF).astype(np.uint8)
    else:
        codes = ((q[0::2] & 0xF) | ((q[1::2] & 0xF) << 4)).astype(np.uint8)
    return codes, s.astype(np.float32)


def np_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    if bits == 8:
        return codes.view(np.int8).astype(np.int64)
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    q = np.stack([lo, hi], axis=1).reshape(-1)
    return np.where(q >= 8, q - 16, q)


def np_dequantize(codes, scales, bits, block):
    return np_codes(codes, bits).astype(np.float32) * np.repeat(scales, block)


def np_sum(codes_list, scales_list, bits, block):
    acc = None
    for c, s in zip(codes_list, scales_list):
        p = np_dequantize(c, s, bits, block)
        acc = (np.float32(0) + p) if acc is None else acc + p  # acc = +0 + p first, as the oracle
    return acc


def np_reorder(buf: np.ndarray, n: int, g: int) -> np.ndarray:
    N = n * g
    sl = buf.reshape(N, -1)
    out = np.empty_like(sl)
    for j in range(g):
        for k in range(n):
            out[j * n + k] = sl[k * g + j]
    return out.reshape(-1)


def _inputs(kind: str, n: int, seed: int):
    rng = np.random.default_rng([31, seed])
    if kind == "bf16":
        x = rng.standard_normal(n).astype(np.float32) * np.exp(rng.uniform(-40, 40, n // 64)).astype(
            np.float32).repeat(64)
        x[::97] = 0.0
        x[64:128] = 0.0                                             # an all-zero block (B <= 64)
        bits = (x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16
        return bits.astype(np.uint16)
    x = rng.standard_normal(n).astype(np.float32) * np.exp(rng.uniform(-80, 80, n // 64)).astype(np.float32).repeat(64)
    x[:64] *= np.float32(1e-37)                                      # subnormal and underflowing scales
    return x


@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("block", [32, 64, 256, 4096])
def test_quantize_and_dequantize_agree(oracle_lib, kind, bits, block):
    x = _inputs(kind, 8192, block + bits)
    c1, s1 = oracle.quantize(x, block, bits)
    c2, s2 = np_quantize(x, block, bits)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(c1, c2)
    y1 = oracle.dequantize(c1, s1, bits, x.size, block)
    y2 = np_dequantize(c2, s2, bits, block)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("bits_in,bits_out", [(4, 4), (8, 8), (4, 0)])
@pytest.mark.parametrize("R", [1, 3, 8])
def test_hop_sum_requant_and_average_agree(oracle_lib, bits_in, bits_out, R):
    block, n = 128, 4096
    pieces = [np_quantize(_inputs("f32", n, 100 + r), block, bits_in) for r in range(R)]
    cl, sl = [p[0] for p in pieces], [p[1] for p in pieces]
    co, so, su = oracle.dequant_reduce_requant(cl, sl, bits_in, n, block, bits_out)
    s2 = np_sum(cl, sl, bits_in, block)
    assert np.array_equal(su.view(np.uint32), s2.view(np.uint32))
    if bits_out:
        c2, q2 = np_quantize(s2, block, bits_out)
        assert np.array_equal(co, c2) and np.array_equal(so.view(np.uint32), q2.view(np.uint32))
    for d in (3, 256):
        avg = oracle.dequant_average(cl, sl, bits_in, n, block, d)
        assert np.array_equal(avg.view(np.uint32), (s2 / np.float32(d)).view(np.uint32))


@pytest.mark.parametrize("n,g", [(2, 4), (4, 2), (3, 5), (1, 4), (4, 1)])
def test_reorder_agrees(oracle_lib, n, g):
    buf = np.random.default_rng([n, g]).integers(0, 1 << 16, n * g * 40, dtype=np.uint16)
    assert np.array_equal(oracle.reorder_slices(buf, n, g), np_reorder(buf, n, g))
