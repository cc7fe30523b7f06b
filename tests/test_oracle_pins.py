"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against a hand-derived worked example, an exact
rational computation (``fractions.Fraction``), a library routine, or an
invariant that symmetric block quantization must satisfy. Sources: page
"Quantized LLM Training at Scale with ZeRO++", section "The Three Pillars of
ZeRO++" (QWZ block quantization to 8 bits with better precision than global
quantization; QGZ 4-bit one-shot quantization and the hop reduction), and
the readings in ``oracle/zpp_oracle.c``.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
QMAX = {8: 127, 4: 7}


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_from_hex(hs):
    return np.array([int(h, 16) for h in hs], dtype=np.uint32).view(np.float32)


def _bf16_bits(vals):
    return synth._f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _codes_int(codes: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Decode code bytes to integers (two's complement; low nibble first)."""
    if bits == 8:
        return codes.view(np.int8).astype(np.int64)[:n]
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    q = np.empty(2 * codes.size, dtype=np.int64)
    q[0::2] = lo
    q[1::2] = hi
    q = np.where(q >= 8, q - 16, q)
    return q[:n]


def _pack(q, bits):
    q = np.asarray(q, dtype=np.int64)
    if bits == 8:
        return (q & 0xFF).astype(np.uint8)
    q = q & 0xF
    return (q[0::2] | (q[1::2] << 4)).astype(np.uint8)


# --------------------------------------------------------------------------
# hand-derived worked examples
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("quantize_cases.json")["cases"], ids=lambda c: c["name"])
def test_golden_quantize(oracle_lib, case):
    if "x_bits_hex" in case:
        x = _f32_from_hex(case["x_bits_hex"])
    else:
        x = np.asarray(case["x"], dtype=np.float32)
    if case["dtype"] == "bf16":
        xin = _bf16_bits(x)
        assert np.array_equal(oracle.bf16_decode(xin), x), "golden input not exact in bf16"
    else:
        xin = x
    codes, scales = oracle.quantize(xin, case["block"], case["bits"])
    assert codes.tobytes().hex() == case["codes_hex"]
    if "scales_bits_hex" in case:
        assert scales.view(np.uint32).tolist() == [int(h, 16) for h in case["scales_bits_hex"]]
    else:
        assert scales.tolist() == case["scales"]


@pytest.mark.parametrize("case", _load("dequantize_cases.json")["cases"], ids=lambda c: c["name"])
def test_golden_dequantize(oracle_lib, case):
    codes = np.frombuffer(bytes.fromhex(case["codes_hex"]), dtype=np.uint8)
    if "scales_bits_hex" in case:
        scales = _f32_from_hex(case["scales_bits_hex"])
    else:
        scales = np.asarray(case["scales"], dtype=np.float32)
    n = codes.size * 8 // case["bits"]
    if "y_f32" in case:
        y = oracle.dequantize(codes, scales, case["bits"], n, case["block"], out="f32")
        assert y.tolist() == case["y_f32"]
    if "y_bf16_hex" in case:
        y = oracle.dequantize(codes, scales, case["bits"], n, case["block"], out="bf16")
        assert [f"{v:04x}" for v in y.tolist()] == case["y_bf16_hex"]


@pytest.mark.parametrize("case", _load("reduce_cases.json")["cases"], ids=lambda c: c["name"])
def test_golden_reduce(oracle_lib, case):
    codes, scales = [], []
    for inp in case["inputs"]:
        codes.append(_pack(inp["codes"], case["bits_in"]))
        if "scales_bits_hex" in inp:
            scales.append(_f32_from_hex(inp["scales_bits_hex"]))
        else:
            scales.append(np.asarray(inp["scales"], dtype=np.float32))
    n = len(case["inputs"][0]["codes"])
    co, so, total = oracle.dequant_reduce_requant(codes, scales, case["bits_in"], n, case["block"],
                                                  case["bits_out"])
    assert total.tolist() == case["sum"]
    if "sum_bits_hex" in case:  # == cannot tell -0 from +0: compare the bit patterns
        assert [f"{v:08x}" for v in total.view(np.uint32).tolist()] == case["sum_bits_hex"]
    assert so.tolist() == case["out_scales"]
    assert _codes_int(co, case["bits_out"], n).tolist() == case["out_codes"]


# --------------------------------------------------------------------------
# exact-arithmetic checks
# --------------------------------------------------------------------------

def _special_blocks(block: int) -> np.ndarray:
    """bf16 blocks exercising ties, extremes and subnormals (as float32 values)."""
    rng = np.random.default_rng([7, block])
    out = []
    # integer-valued halves relative to a power-of-two scale: lots of exact ties
    for Q in (127, 7):
        b = rng.integers(-2 * Q, 2 * Q + 1, block).astype(np.float32) / 2
        b[0] = Q
        out.append(b)
    # max finite bfloat16 and smallest subnormal bfloat16 absmax
    big = np.float32(np.uint32(0x7F7F0000).view(np.float32))
    b = rng.standard_normal(block).astype(np.float32) * (big / np.float32(8))
    b[1] = -big
    out.append(b)
    tiny = np.uint32(0x00010000).view(np.float32)  # bf16 0x0001 = 2^-133
    b = (rng.integers(-1, 2, block) * tiny).astype(np.float32)
    b[2] = tiny
    out.append(b)
    sub = np.uint32(0x00400000).view(np.float32)  # 2^-127 (subnormal)
    b = (rng.integers(-3, 4, block) * sub).astype(np.float32)
    out.append(b)
    out.append(np.zeros(block, np.float32))
    return np.concatenate(out)


def _random_bf16_blocks(block: int, nblocks: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([11, block, seed])
    x = rng.standard_normal(block * nblocks).astype(np.float32)
    x *= np.exp(rng.uniform(-30, 30, nblocks)).astype(np.float32).repeat(block)
    return x


def _nearest_f32(value: Fraction, got: np.float32) -> bool:
    """True when ``got`` is a binary32 nearest to ``value`` (ties: even mantissa)."""
    g = Fraction(float(got))
    lo = Fraction(float(np.nextafter(got, np.float32(-np.inf))))
    hi = Fraction(float(np.nextafter(got, np.float32(np.inf))))
    d = abs(g - value)
    if d > abs(lo - value) or d > abs(hi - value):
        return False
    if d == abs(lo - value) or d == abs(hi - value):
        return int(np.float32(got).view(np.uint32)) % 2 == 0
    return True


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("block", [32, 256])
def test_scale_is_correctly_rounded_absmax_over_q(oracle_lib, bits, block):
    x = np.concatenate([_special_blocks(block), _random_bf16_blocks(block, 64, bits)])
    xb = synth._f32_to_bf16_bits(x)
    xv = oracle.bf16_decode(xb)
    _, scales = oracle.quantize(xb, block, bits)
    Q = QMAX[bits]
    for b in range(xv.size // block):
        a = np.abs(xv[b * block:(b + 1) * block]).max()
        assert _nearest_f32(Fraction(float(a)) / Q, scales[b]), (b, a, scales[b])


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("block", [32, 128])
def test_codes_are_nearest_grid_points(oracle_lib, bits, block):
    """Each code is the integer nearest x/s (exact rational), ties to even, clamped to [-Q, Q]."""
    x = np.concatenate([_special_blocks(block), _random_bf16_blocks(block, 24, 100 + bits)])
    xb = synth._f32_to_bf16_bits(x)
    xv = oracle.bf16_decode(xb)
    codes, scales = oracle.quantize(xb, block, bits)
    q = _codes_int(codes, bits, xv.size)
    Q = QMAX[bits]
    # The reading rounds the binary32 quotient fl(x/s) first, then to an integer,
    # so x/s within half an ulp of a half-integer may land on the tie itself.
    slack = Fraction(1, 1 << 16)
    for i in range(xv.size):
        s = scales[i // block]
        if s == 0:
            assert q[i] == 0
            continue
        R = Fraction(float(xv[i])) / Fraction(float(s))
        assert -Q <= q[i] <= Q
        if R > Q + Fraction(1, 2) + slack:
            assert q[i] == Q
            continue
        if R < -Q - Fraction(1, 2) - slack:
            assert q[i] == -Q
            continue
        dist = abs(R - q[i])
        if dist > Fraction(1, 2):
            # allowed only when fl(x/s) rounded onto the half-integer next to q
            # and the tie went to the even integer
            half = q[i] + (Fraction(1, 2) if R > q[i] else Fraction(-1, 2))
            assert abs(R - half) <= abs(R) / (1 << 24), (i, float(R), q[i])
            assert q[i] % 2 == 0, (i, float(R), q[i])
        elif dist == Fraction(1, 2):  # exact tie: must be even
            assert q[i] % 2 == 0, (i, float(R), q[i])


@pytest.mark.parametrize("bits", [8, 4])
def test_dequantized_value_is_rounded_exact_product(oracle_lib, bits):
    rng = np.random.default_rng(3)
    block = 64
    n = block * 40
    codes = rng.integers(0, 256, n * bits // 8, dtype=np.uint8)
    scales = np.exp(rng.uniform(-80, 80, n // block)).astype(np.float32)
    scales[0] = np.uint32(0x00000321).view(np.float32)  # subnormal scale
    y = oracle.dequantize(codes, scales, bits, n, block, out="f32")
    q = _codes_int(codes, bits, n)
    for i in range(n):
        exact = q[i] * Fraction(float(scales[i // block]))
        assert _nearest_f32(exact, y[i]), (i, q[i], scales[i // block], y[i])
    yb = oracle.dequantize(codes, scales, bits, n, block, out="bf16")
    import torch
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, ref)


def test_bf16_rounding_matches_library_cast(oracle_lib):
    """The oracle's binary32 -> bfloat16 rounding agrees with torch's cast, ties and subnormals included."""
    import torch
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    u[:50_000] = (u[:50_000] & 0xFFFF0000) | 0x8000  # exact ties
    u[50_000:60_000] &= 0x807FFFFF  # subnormals
    u = u[(u & 0x7F800000) != 0x7F800000]  # drop inf/nan
    x = u.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(x), ref)


def test_bf16_decode_is_exact(oracle_lib):
    import torch
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    h = h[(h & 0x7F80) != 0x7F80]
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_decode(h).view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def _workload_like(n, kind, seed):
    if kind == "qwz":     # N(0, 0.02) with 0.1 % outliers x50
        return synth.small_bf16(n, (seed, 1), 0.02, 1e-3, 50.0)
    if kind == "gqa":     # N(0, 0.01) with 0.01 % outliers x100
        return synth.small_bf16(n, (seed, 5), 0.01, 1e-4, 100.0)
    if kind == "grad":    # N(0, 1e-3)
        return synth.small_bf16(n, (seed, 2), 1e-3)
    if kind == "t3":      # Student-t(3) x 1e-4
        return synth.bf16_student_t(n, 3.0, 1e-4, (seed, 4))
    raise ValueError(kind)


@pytest.mark.parametrize("bits,block,kind", [(8, 256, "qwz"), (8, 512, "gqa"), (4, 128, "grad"),
                                             (4, 256, "t3"), (4, 128, "gqa"), (8, 2048, "qwz")])
def test_error_at_most_half_scale(oracle_lib, bits, block, kind):
    """|x - dequant(quant(x))| <= s/2 plus binary32 rounding of the quotient and product."""
    xb = _workload_like(1 << 18, kind, 0)
    x = oracle.bf16_decode(xb).astype(np.float64)
    codes, scales = oracle.quantize(xb, block, bits)
    y = oracle.dequantize(codes, scales, bits, xb.size, block, out="f32").astype(np.float64)
    s = np.repeat(scales.astype(np.float64), block)
    err = np.abs(x - y)
    assert np.all(err <= s * (0.5 + 2.0 ** -15)), float(np.max(err / np.maximum(s, 1e-45)))
    # the bound is tight: some element comes close to s/2
    assert np.max(err / np.where(s > 0, s, 1)) > 0.49


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128), (8, 32), (4, 4096)])
def test_absmax_element_gets_full_scale_code(oracle_lib, bits, block):
    xb = _workload_like(1 << 17, "qwz", 1)
    x = oracle.bf16_decode(xb).reshape(-1, block)
    codes, scales = oracle.quantize(xb, block, bits)
    q = _codes_int(codes, bits, xb.size).reshape(-1, block)
    Q = QMAX[bits]
    assert np.all(np.abs(q) <= Q)
    idx = np.argmax(np.abs(x), axis=1)
    rows = np.arange(x.shape[0])
    nz = scales > 0
    assert np.all(np.abs(q[rows, idx])[nz] == Q)
    assert np.all(np.sign(q[rows, idx])[nz] == np.sign(x[rows, idx])[nz])


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_negation_symmetry(oracle_lib, bits, block):
    xb = _workload_like(1 << 16, "grad", 2)
    codes, scales = oracle.quantize(xb, block, bits)
    ncodes, nscales = oracle.quantize(xb ^ np.uint16(0x8000), block, bits)
    assert np.array_equal(scales, nscales)
    assert np.array_equal(_codes_int(ncodes, bits, xb.size), -_codes_int(codes, bits, xb.size))


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128), (4, 32)])
def test_requantizing_dequantized_values_keeps_codes(oracle_lib, bits, block):
    xb = _workload_like(1 << 16, "t3", 3)
    codes, scales = oracle.quantize(xb, block, bits)
    y = oracle.dequantize(codes, scales, bits, xb.size, block, out="f32")
    codes2, scales2 = oracle.quantize(y, block, bits)
    assert np.array_equal(codes2, codes)
    # the scale may move by at most one ulp (a/Q is rounded twice)
    ulp = np.abs(np.nextafter(scales, np.float32(np.inf)) - scales)
    assert np.all(np.abs(scales2 - scales) <= ulp)


@pytest.mark.parametrize("k", [-12, -1, 1, 7])
@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_power_of_two_scaling(oracle_lib, bits, block, k):
    """Scaling x by 2^k leaves the codes alone and scales every s by exactly 2^k."""
    xb = _workload_like(1 << 16, "grad", 4)
    x = oracle.bf16_decode(xb)
    xs = (x * np.float32(2.0 ** k)).astype(np.float32)
    xsb = oracle.bf16_round(xs)
    assert np.array_equal(oracle.bf16_decode(xsb), xs)  # exact scaling in bf16
    codes, scales = oracle.quantize(xb, block, bits)
    codes2, scales2 = oracle.quantize(xsb, block, bits)
    assert np.array_equal(codes, codes2)
    assert np.array_equal(scales2, (scales * np.float32(2.0 ** k)).astype(np.float32))


@pytest.mark.parametrize("kind,bits,block", [("qwz", 8, 256), ("gqa", 8, 512), ("grad", 4, 128)])
def test_block_quantization_beats_global(oracle_lib, kind, bits, block):
    """Per-block scales give lower squared error than one scale for the whole tensor.

    Not a theorem (integer data with absmax Q breaks it); checked on the
    workloads' own distributions. The ratio is reported next to the 3.3x
    precision gain the ZeRO++ page quotes for QWZ (metric unstated there, so
    the figure itself is not pinned).
    """
    xb = _workload_like(1 << 18, kind, 5)
    x = oracle.bf16_decode(xb).astype(np.float64)
    cb, sb = oracle.quantize(xb, block, bits)
    cg, sg = oracle.quantize(xb, xb.size, bits)
    yb = oracle.dequantize(cb, sb, bits, xb.size, block).astype(np.float64)
    yg = oracle.dequantize(cg, sg, bits, xb.size, xb.size).astype(np.float64)
    mse_b = np.mean((x - yb) ** 2)
    mse_g = np.mean((x - yg) ** 2)
    assert mse_b < mse_g
    print(f"{kind} int{bits} B={block}: global/block RMS error = {np.sqrt(mse_g / mse_b):.2f}")


def test_sizes_halve_and_quarter_the_volume(oracle_lib):
    """8-bit codes are half the bf16 bytes, 4-bit a quarter, plus 4 bytes of scale per block
    (the M -> 0.5M and M -> 0.25M volumes of QWZ and QGZ)."""
    for n, block in [(4096 * 4096, 256), (16_000_000, 128), (1 << 20, 2048)]:
        xb = np.zeros(n, np.uint16) if n <= (1 << 20) else None
        for bits, ratio in [(8, 0.5), (4, 0.25)]:
            assert oracle.codes_nbytes(n, bits) == ratio * 2 * n
            if xb is not None:
                codes, scales = oracle.quantize(xb, block, bits)
                assert codes.nbytes == ratio * xb.nbytes
                assert scales.nbytes == 4 * n // block


# --------------------------------------------------------------------------
# the hop reduction
# --------------------------------------------------------------------------

@pytest.mark.parametrize("R", [1, 2, 4, 8, 32])
@pytest.mark.parametrize("bits", [4, 8])
def test_sum_of_small_exact_terms_is_exact(oracle_lib, R, bits):
    """With power-of-two scales every product and partial sum is exact, so the
    oracle's binary32 sum must equal the exact integer-rational sum."""
    rng = np.random.default_rng([R, bits])
    block, n = 32, 32 * 16
    Q = QMAX[bits]
    qs = [rng.integers(-Q, Q + 1, n) for _ in range(R)]
    ss = [np.float32(2.0) ** rng.integers(-4, 5, n // block).astype(np.float32) for _ in range(R)]
    total = oracle.dequant_sum([_pack(q, bits) for q in qs], ss, bits, n, block)
    for i in range(n):
        exact = sum(Fraction(int(qs[r][i])) * Fraction(float(ss[r][i // block])) for r in range(R))
        assert Fraction(float(total[i])) == exact


@pytest.mark.parametrize("R", [2, 8, 32])
def test_sum_within_binary32_error_of_exact(oracle_lib, R):
    rng = np.random.default_rng([R, 99])
    block, n = 128, 128 * 8
    qs = [rng.integers(-7, 8, n) for _ in range(R)]
    ss = [np.exp(rng.uniform(-10, 0, n // block)).astype(np.float32) for _ in range(R)]
    total = oracle.dequant_sum([_pack(q, 4) for q in qs], ss, 4, n, block).astype(np.float64)
    terms = np.stack([qs[r] * np.repeat(ss[r].astype(np.float64), block) for r in range(R)])
    exact = terms.sum(axis=0)
    bound = np.abs(terms).sum(axis=0) * 2.0 ** -23 * R
    assert np.all(np.abs(total - exact) <= bound)


def test_requant_of_hop_sum_obeys_quantizer_pins(oracle_lib):
    """The requantized hop output is a block quantization of the binary32 sum:
    its error against the sum is at most half its scale."""
    rng = np.random.default_rng(12)
    block, n, R = 256, 256 * 32, 8
    xs = [synth.bf16_student_t(n, 3.0, 1e-4, (12, r)) for r in range(R)]
    qs = [oracle.quantize(x, block, 4) for x in xs]
    co, so, total = oracle.dequant_reduce_requant([c for c, _ in qs], [s for _, s in qs], 4, n, block, 4)
    y = oracle.dequantize(co, so, 4, n, block).astype(np.float64)
    s = np.repeat(so.astype(np.float64), block)
    assert np.all(np.abs(y - total) <= s * (0.5 + 2.0 ** -15))
    del rng
