"""Seeded random parity cases for every entry point.

Each case draws its shape and parameters (element count, block size, code
widths, slice grid, input count, strides with gaps, divisor) and its data
(bf16 or fp32 values over many binades with zeros and exact ties; arbitrary
code bytes; scales that are zero, subnormal, negative or large) from a seeded
generator, runs the library through its C ABI on canary-guarded buffers, and
compares every output with the oracle bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import Guarded, assert_bits_equal, dev, need_gpu, torch

pytestmark = pytest.mark.gpu

BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _z():
    import block_quantization_codec_amd as z
    return z


def _values(rng, n: int, block: int) -> np.ndarray:
    """fp32 values, one random binade per block, with zeros and exact ties."""
    nb = n // block
    x = rng.standard_normal(n).astype(np.float32)
    x *= np.exp2(rng.integers(-130, 120, nb)).astype(np.float32).repeat(block)
    x[rng.random(n) < 0.05] = 0.0
    ties = rng.random(n) < 0.05
    x[ties] = (rng.integers(-30, 30, int(ties.sum())) + 0.5).astype(np.float32)
    x[rng.random(n) < 0.01] = -0.0
    x[: block] = 0.0 if rng.random() < 0.5 else x[: block]   # sometimes an all-zero first block
    return x


def _bf16(x: np.ndarray) -> np.ndarray:
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _scales(rng, n: int) -> np.ndarray:
    s = np.exp2(rng.uniform(-140, 100, n)).astype(np.float32)
    kind = rng.random(n)
    s[kind < 0.1] = 0.0
    s[(kind >= 0.1) & (kind < 0.15)] *= -1.0
    return s


@pytest.mark.parametrize("seed", range(96))
def test_random_quantize_and_dequantize(seed):
    z = _z()
    rng = np.random.default_rng([600, seed])
    B = int(rng.choice(BLOCKS))
    bits = int(rng.choice([8, 4]))
    n = B * int(rng.integers(1, max(2, 40000 // B)))
    xf = _values(rng, n, B)
    x = _bf16(xf) if rng.random() < 0.6 else xf
    dt = z.ZPP_BF16 if x.dtype == np.uint16 else z.ZPP_FP32
    gc, gs = Guarded(n * bits // 8), Guarded(4 * (n // B))
    xd = dev(x)
    torch.cuda.synchronize()
    z.zpp_quantize_blocks(xd, dt, n, B, bits, gc.ptr, gs.ptr)
    torch.cuda.synchronize()
    assert gc.untouched() and gs.untouched()
    oc, os_ = oracle.quantize(x, B, bits)
    assert_bits_equal(gc.bytes(), oc, f"codes seed={seed} B={B} bits={bits} n={n}")
    assert_bits_equal(gs.as_np(np.float32), os_, f"scales seed={seed}")
    out_f32 = rng.random() < 0.5
    gy = Guarded(n * (4 if out_f32 else 2))
    codes = dev(rng.integers(0, 256, n * bits // 8, dtype=np.uint8))   # arbitrary code bytes
    scales = _scales(rng, n // B)
    sd = dev(scales)
    torch.cuda.synchronize()
    z.zpp_dequantize_blocks(codes, sd, bits, n, B, gy.ptr, z.ZPP_FP32 if out_f32 else z.ZPP_BF16)
    torch.cuda.synchronize()
    assert gy.untouched()
    oy = oracle.dequantize(codes.cpu().numpy(), scales, bits, n, B, out="f32" if out_f32 else "bf16")
    assert_bits_equal(gy.as_np(np.float32 if out_f32 else np.uint16), oy, f"dequantized seed={seed}")


@pytest.mark.parametrize("seed", range(48))
def test_random_reorder_and_fused_quantize(seed):
    z = _z()
    rng = np.random.default_rng([601, seed])
    n_nodes, g = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    N = n_nodes * g
    B = int(rng.choice(BLOCKS[:5]))
    bits = int(rng.choice([8, 4]))
    S = B * int(rng.integers(1, 12))
    xf = _values(rng, N * S, B)
    x = _bf16(xf) if rng.random() < 0.6 else xf
    dt = z.ZPP_BF16 if x.dtype == np.uint16 else z.ZPP_FP32
    xd = dev(x)
    esz = x.dtype.itemsize
    go = Guarded(N * S * esz)
    torch.cuda.synchronize()
    z.zpp_reorder_slices(xd, go.ptr, S * esz, n_nodes, g)
    torch.cuda.synchronize()
    assert go.untouched()
    ore = oracle.reorder_slices(x, n_nodes, g)
    assert_bits_equal(go.as_np(x.dtype), ore, f"reorder seed={seed} grid={n_nodes}x{g}")
    first = int(rng.integers(0, N))
    count = int(rng.integers(1, N - first + 1))
    gc, gs = Guarded(count * S * bits // 8), Guarded(4 * count * S // B)
    torch.cuda.synchronize()
    z.zpp_quantize_reordered(xd, dt, S, n_nodes, g, first, count, B, bits, gc.ptr, gs.ptr)
    torch.cuda.synchronize()
    assert gc.untouched() and gs.untouched()
    oc, os_ = oracle.quantize(ore[first * S:(first + count) * S], B, bits)
    assert_bits_equal(gc.bytes(), oc, f"fused codes seed={seed}")
    assert_bits_equal(gs.as_np(np.float32), os_, f"fused scales seed={seed}")


@pytest.mark.parametrize("seed", range(96))
def test_random_hop_reduce_and_average(seed):
    z = _z()
    rng = np.random.default_rng([602, seed])
    B = int(rng.choice(BLOCKS))
    bits_in = int(rng.choice([8, 4]))
    bits_out = int(rng.choice([0, 4, 8]))
    R = int(rng.integers(1, 40))
    n = B * int(rng.integers(1, max(2, 20000 // B)))
    gap_blocks = int(rng.integers(0, 3))
    per_c = (n + gap_blocks * B) * bits_in // 8
    per_c += (-per_c) % 16                                   # strides are multiples of 16 bytes
    per_s = n // B + gap_blocks
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    if rng.random() < 0.5:                                   # or codes of real quantized data
        for r in range(R):
            c, s = oracle.quantize(_values(rng, n, B), B, bits_in)
            codes[r * per_c:r * per_c + c.size] = c
    scales = _scales(rng, R * per_s)
    if rng.random() < 0.5:
        scales = np.abs(scales)
    cl = [codes[r * per_c:r * per_c + n * bits_in // 8] for r in range(R)]
    sl = [scales[r * per_s:r * per_s + n // B] for r in range(R)]
    cd, sd = dev(codes), dev(scales)
    want_sum = bits_out == 0 or rng.random() < 0.5
    gc = Guarded(n * bits_out // 8) if bits_out else None
    gs = Guarded(4 * (n // B)) if bits_out else None
    gu = Guarded(4 * n) if want_sum else None
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_requant(cd, per_c, sd, per_s, R, bits_in, n, B, gc.ptr if gc else None,
                                 gs.ptr if gs else None, bits_out, gu.ptr if gu else None)
    torch.cuda.synchronize()
    co, so, su = oracle.dequant_reduce_requant(cl, sl, bits_in, n, B, bits_out)
    finite = np.isfinite(su).all()
    if gu is not None:
        assert gu.untouched()
        assert_bits_equal(gu.as_np(np.float32), su, f"sum seed={seed} B={B} R={R} {bits_in}->{bits_out}")
    if bits_out and finite:  # a sum that overflows is outside the requantization contract
        assert gc.untouched() and gs.untouched()
        assert_bits_equal(gs.as_np(np.float32), so, f"requantized scales seed={seed}")
        assert_bits_equal(gc.bytes(), co, f"requantized codes seed={seed}")
    if bits_out and finite:  # the same hop with its output split at a random kept window of blocks
        nb = n // B
        k0 = int(rng.integers(0, nb + 1))
        kl = int(rng.integers(0, nb - k0 + 1))
        k0, kl = k0 * B, kl * B
        gsc = Guarded((n - kl) * bits_out // 8) if n > kl else None
        gss = Guarded(4 * ((n - kl) // B)) if n > kl else None
        gkc = Guarded(kl * bits_out // 8) if kl else None
        gks = Guarded(4 * (kl // B)) if kl else None
        torch.cuda.synchronize()
        z.zpp_dequant_reduce_requant_split(cd, per_c, sd, per_s, R, bits_in, n, B, k0, kl,
                                           gsc.ptr if gsc else None, gss.ptr if gss else None,
                                           gkc.ptr if gkc else None, gks.ptr if gks else None, bits_out)
        torch.cuda.synchronize()
        cb = bits_out // 8 if bits_out == 8 else 0.5
        c0, c1 = int(k0 * cb), int((k0 + kl) * cb)
        if kl:
            assert gkc.untouched() and gks.untouched()
            assert_bits_equal(gkc.bytes(), co[c0:c1], f"split kept codes seed={seed}")
            assert_bits_equal(gks.as_np(np.float32), so[k0 // B:(k0 + kl) // B], f"split kept scales seed={seed}")
        if n > kl:
            assert gsc.untouched() and gss.untouched()
            assert_bits_equal(gsc.bytes(), np.concatenate([co[:c0], co[c1:]]), f"split sent codes seed={seed}")
            assert_bits_equal(gss.as_np(np.float32), np.concatenate([so[:k0 // B], so[(k0 + kl) // B:]]),
                              f"split sent scales seed={seed}")
    divisor = int(rng.choice([1, 3, 7, 8, 96, 1 << 20]))
    ga = Guarded(4 * n)
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_average(cd, per_c, sd, per_s, R, bits_in, n, B, divisor, ga.ptr)
    torch.cuda.synchronize()
    assert ga.untouched()
    assert_bits_equal(ga.as_np(np.float32), oracle.dequant_average(cl, sl, bits_in, n, B, divisor),
                      f"average seed={seed} divisor={divisor}")


@pytest.mark.parametrize("seed", range(24))
def test_random_wide_hops(seed):
    """Random hops large enough for the 32-elements-per-lane layouts: the
    LDS-staged one (4-bit inputs, blocks up to 2048; from 1,536 waves with at
    most 4 inputs, else from 4,096) and the register one (8-bit inputs, and
    4,096-element blocks), with random input counts, strides with gaps, code
    bytes, scales across binades and a random kept window for the split."""
    import oracle_par
    z = _z()
    rng = np.random.default_rng([603, seed])
    bits_in = int(rng.choice([4, 4, 8]))
    B = int(rng.choice([32, 128, 256, 512, 2048, 4096]))
    R = int(rng.integers(1, 13))
    waves = int(rng.integers(1536 if (bits_in == 4 and R <= 4) else 4096, 4600))
    n = (waves * 2048 - int(rng.integers(0, 2048))) // B * B
    bits_out = int(rng.choice([4, 8]))
    gap_blocks = int(rng.integers(0, 3))
    per_c = (n + gap_blocks * B) * bits_in // 8
    per_c += (-per_c) % 16
    per_s = n // B + gap_blocks
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    scales = np.exp2(rng.uniform(-30, 10, R * per_s)).astype(np.float32)
    scales[rng.random(scales.size) < 0.02] = 0.0
    cl = [codes[r * per_c:r * per_c + n * bits_in // 8] for r in range(R)]
    sl = [scales[r * per_s:r * per_s + n // B] for r in range(R)]
    cd, sd = dev(codes), dev(scales)
    co, so, su = oracle_par.dequant_reduce_requant(cl, sl, bits_in, n, B, bits_out)
    what = f"seed={seed} B={B} R={R} n={n} {bits_in}->{bits_out}"
    gc, gs, gu = Guarded(n * bits_out // 8), Guarded(4 * (n // B)), Guarded(4 * n)
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_requant(cd, per_c, sd, per_s, R, bits_in, n, B, gc.ptr, gs.ptr, bits_out, gu.ptr)
    torch.cuda.synchronize()
    assert gc.untouched() and gs.untouched() and gu.untouched()
    assert_bits_equal(gu.as_np(np.float32), su, "sum " + what)
    assert_bits_equal(gs.as_np(np.float32), so, "scales " + what)
    assert_bits_equal(gc.bytes(), co, "codes " + what)
    nb = n // B
    k0 = int(rng.integers(0, nb + 1))
    kl = int(rng.integers(0, nb - k0 + 1))
    k0, kl = k0 * B, kl * B
    gsc = Guarded((n - kl) * bits_out // 8) if n > kl else None
    gss = Guarded(4 * ((n - kl) // B)) if n > kl else None
    gkc = Guarded(kl * bits_out // 8) if kl else None
    gks = Guarded(4 * (kl // B)) if kl else None
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_requant_split(cd, per_c, sd, per_s, R, bits_in, n, B, k0, kl,
                                       gsc.ptr if gsc else None, gss.ptr if gss else None,
                                       gkc.ptr if gkc else None, gks.ptr if gks else None, bits_out)
    torch.cuda.synchronize()
    cb = bits_out / 8
    c0, c1 = int(k0 * cb), int((k0 + kl) * cb)
    if kl:
        assert gkc.untouched() and gks.untouched()
        assert_bits_equal(gkc.bytes(), co[c0:c1], "split kept codes " + what)
        assert_bits_equal(gks.as_np(np.float32), so[k0 // B:(k0 + kl) // B], "split kept scales " + what)
    if n > kl:
        assert gsc.untouched() and gss.untouched()
        assert_bits_equal(gsc.bytes(), np.concatenate([co[:c0], co[c1:]]), "split sent codes " + what)
        assert_bits_equal(gss.as_np(np.float32), np.concatenate([so[:k0 // B], so[(k0 + kl) // B:]]),
                          "split sent scales " + what)


@pytest.mark.parametrize("seed", range(16))
def test_random_wide_sums(seed):
    """Random hops of the 32-elements-per-lane layouts that write only binary32
    sums or averages (the last hop), whose sums go out through LDS so that each
    store is contiguous across the wave: the LDS-staged layout (4-bit inputs,
    blocks up to 2048) reuses its code slots for them, the register layout
    (8-bit inputs, 4,096-element blocks) has its own. Random input counts,
    strides with gaps, scales across binades, a ragged end, random divisors."""
    import oracle_par
    z = _z()
    rng = np.random.default_rng([604, seed])
    bits_in = int(rng.choice([4, 8]))
    B = int(rng.choice([32, 128, 256, 1024, 2048, 4096]))
    R = int(rng.integers(1, 40))
    waves = int(rng.integers(1536 if (bits_in == 4 and R <= 4) else 4096, 4600))
    n = (waves * 2048 - int(rng.integers(0, 2048))) // B * B
    gap_blocks = int(rng.integers(0, 3))
    per_c = (n + gap_blocks * B) * bits_in // 8
    per_c += (-per_c) % 16
    per_s = n // B + gap_blocks
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    scales = np.exp2(rng.uniform(-30, 10, R * per_s)).astype(np.float32)
    scales[rng.random(scales.size) < 0.02] = 0.0
    cl = [codes[r * per_c:r * per_c + n * bits_in // 8] for r in range(R)]
    sl = [scales[r * per_s:r * per_s + n // B] for r in range(R)]
    cd, sd = dev(codes), dev(scales)
    what = f"seed={seed} B={B} R={R} n={n} bits={bits_in}"
    _, _, su = oracle_par.dequant_reduce_requant(cl, sl, bits_in, n, B, 0)
    gu = Guarded(4 * n)
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_requant(cd, per_c, sd, per_s, R, bits_in, n, B, None, None, 0, gu.ptr)
    torch.cuda.synchronize()
    assert gu.untouched()
    assert_bits_equal(gu.as_np(np.float32), su, "sum " + what)
    divisor = int(rng.choice([3, 7, 96, 256, 1 << 20]))
    ga = Guarded(4 * n)
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_average(cd, per_c, sd, per_s, R, bits_in, n, B, divisor, ga.ptr)
    torch.cuda.synchronize()
    assert ga.untouched()
    assert_bits_equal(ga.as_np(np.float32), oracle.dequant_average(cl, sl, bits_in, n, B, divisor),
                      f"average {what} divisor={divisor}")
