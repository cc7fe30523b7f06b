"""GPU parity of zpp_dequant_reduce_requant and zpp_dequant_reduce_average
against the CPU oracle.

Codes and scales of the requantized sum must match bit for bit; the binary32
sum must be within 1e-5 of the largest input scale of its block (and is
expected bit-exact, both sides adding the same rounded terms in the same
order). Covers 1..33 inputs (batches of four and remainders), 4- and 8-bit
inputs and outputs, every block size, strided inputs with gaps, the
hand-derived golden cases (order of summation, no fused multiply-add), and
inputs quantized from workload-like data. The averaged variant must match
the oracle bit for bit for odd, even and power-of-two divisors up to 2^24.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import oracle_par
import synth
from gpu_util import Guarded, assert_bits_equal, assert_within_scale, dev, need_gpu, torch

pytestmark = pytest.mark.gpu

BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _run(codes_np, cstride, scales_np, sstride, R, bits_in, numel, block, bits_out, want_sum=True):
    """codes_np / scales_np hold R inputs at the given strides (bytes / floats)."""
    import block_quantization_codec_amd as z
    ci = dev(codes_np)
    si = dev(scales_np)
    gc = Guarded(numel * bits_out // 8) if bits_out else None
    gs = Guarded(4 * (numel // block)) if bits_out else None
    gu = Guarded(4 * numel) if want_sum else None
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_requant(ci, cstride, si, sstride, R, bits_in, numel, block,
                                 gc.ptr if gc else None, gs.ptr if gs else None, bits_out,
                                 gu.ptr if gu else None)
    torch.cuda.synchronize()
    for g in (gc, gs, gu):
        if g is not None:
            assert g.untouched(), "write outside an output buffer"
    return (gc.bytes() if gc else None, gs.as_np(np.float32) if gs else None,
            gu.as_np(np.float32) if gu else None)


def _inputs(R, bits_in, numel, block, seed, gap=0):
    """R inputs quantized (by the oracle) from Student-t data of varying magnitude,
    laid side by side with `gap` spare blocks between them."""
    per_c = numel * bits_in // 8 + gap * block * bits_in // 8
    per_s = numel // block + gap
    codes = np.zeros(R * per_c, np.uint8)
    scales = np.zeros(R * per_s, np.float32)
    for r in range(R):
        x = synth.bf16_student_t(numel, 3.0, 1e-4 * (1 + r % 3), (seed, r, numel, block))
        c, s = oracle.quantize(x, block, bits_in)
        codes[r * per_c:r * per_c + c.size] = c
        scales[r * per_s:r * per_s + s.size] = s
        if gap:
            codes[r * per_c + c.size:(r + 1) * per_c] = 0xEE  # garbage the kernel must not read
            scales[r * per_s + s.size:(r + 1) * per_s] = np.float32(7e30)
    return codes, per_c, scales, per_s


def _expect(codes, per_c, scales, per_s, R, bits_in, numel, block, bits_out):
    cl = [codes[r * per_c:r * per_c + numel * bits_in // 8] for r in range(R)]
    sl = [scales[r * per_s:r * per_s + numel // block] for r in range(R)]
    co, so, su = oracle.dequant_reduce_requant(cl, sl, bits_in, numel, block, bits_out)
    smax = np.max(np.stack(sl), axis=0)
    return co, so, su, np.repeat(smax, block)


def _check(R, bits_in, bits_out, block, numel, seed, gap=0, want_sum=True):
    codes, pc, scales, ps = _inputs(R, bits_in, numel, block, seed, gap)
    gco, gso, gsu = _run(codes, pc, scales, ps, R, bits_in, numel, block, bits_out, want_sum)
    co, so, su, smax = _expect(codes, pc, scales, ps, R, bits_in, numel, block, bits_out)
    what = f"R={R} in={bits_in} out={bits_out} B={block} n={numel}"
    if want_sum:
        assert_within_scale(gsu, su, smax, "sum " + what)
        assert_bits_equal(gsu, su, "sum bits " + what)
    if bits_out:
        assert_bits_equal(gso, so, "scales " + what)
        assert_bits_equal(gco, co, "codes " + what)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 15, 32, 33, 34, 35])
@pytest.mark.parametrize("bits_in,bits_out", [(4, 4), (8, 8), (4, 0)])
def test_input_counts(R, bits_in, bits_out):
    """Every way the 8-elements-per-lane layout splits its inputs: batches of
    8 (the next one loading while the last is summed), then of 4, then the
    last 1, 2 or 3 as one batch."""
    _check(R, bits_in, bits_out, 256, 256 * 100, 1)


@pytest.mark.parametrize("R", [257, 4096])
@pytest.mark.parametrize("bits_in,bits_out", [(4, 4), (8, 0)])
def test_many_inputs(R, bits_in, bits_out):
    """Up to the largest input count the entry point accepts (4096): many
    overlapped batches of 8, then the batch of 4 and single inputs."""
    _check(R, bits_in, bits_out, 256, 256 * 3, 7)


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("bits_in,bits_out", [(4, 4), (8, 8), (4, 8), (8, 4)])
def test_block_sizes(block, bits_in, bits_out):
    nb = max(2, 20_000 // block) + 1
    _check(4, bits_in, bits_out, block, block * nb, 2)


@pytest.mark.parametrize("bits_in,bits_out", [(4, 4), (8, 8)])
def test_strided_inputs_with_gaps(bits_in, bits_out):
    _check(5, bits_in, bits_out, 128, 128 * 333, 3, gap=7)


def test_requant_only_without_sum():
    _check(8, 4, 4, 256, 256 * 64, 4, want_sum=False)


def test_random_code_bytes_and_scales():
    """Arbitrary code patterns (including -8) and scales across binades."""
    rng = np.random.default_rng(5)
    R, block, numel = 6, 64, 64 * 300
    codes = rng.integers(0, 256, R * numel // 2, dtype=np.uint8)
    scales = np.exp2(rng.uniform(-30, 30, R * numel // block)).astype(np.float32)
    gco, gso, gsu = _run(codes, numel // 2, scales, numel // block, R, 4, numel, block, 4)
    cl = [codes[r * numel // 2:(r + 1) * numel // 2] for r in range(R)]
    sl = [scales[r * numel // block:(r + 1) * numel // block] for r in range(R)]
    co, so, su = oracle.dequant_reduce_requant(cl, sl, 4, numel, block, 4)
    assert_bits_equal(gsu, su, "sum")
    assert_bits_equal(gso, so, "scales")
    assert_bits_equal(gco, co, "codes")


def _pack(q, bits):
    q = np.asarray(q, dtype=np.int64)
    if bits == 8:
        return (q & 0xFF).astype(np.uint8)
    q = q & 0xF
    return (q[0::2] | (q[1::2] << 4)).astype(np.uint8)


def test_golden_reduce_cases_on_gpu():
    """Hand-derived cases (blocks of 4) padded with zero codes to a block of 32."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "reduce_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        bi, bo, R = c["bits_in"], c["bits_out"], len(c["inputs"])
        codes = np.zeros(R * 32 * bi // 8, np.uint8)
        scales = np.zeros(R, np.float32)
        for r, inp in enumerate(c["inputs"]):
            q = np.zeros(32, np.int64)
            q[:4] = inp["codes"]
            codes[r * 32 * bi // 8:(r + 1) * 32 * bi // 8] = _pack(q, bi)
            if "scales_bits_hex" in inp:
                scales[r] = np.array([int(inp["scales_bits_hex"][0], 16)], np.uint32).view(np.float32)[0]
            else:
                scales[r] = inp["scales"][0]
        gco, gso, gsu = _run(codes, 32 * bi // 8, scales, 1, R, bi, 32, 32, bo)
        assert gsu[:4].tolist() == c["sum"], c["name"]
        if "sum_bits_hex" in c:  # == cannot tell -0 from +0: compare the bit patterns
            assert [f"{v:08x}" for v in gsu[:4].view(np.uint32).tolist()] == c["sum_bits_hex"], c["name"]
        assert (gsu[4:].view(np.uint32) == 0).all(), c["name"]   # zero padding sums to +0
        assert gso.tolist() == c["out_scales"], c["name"]
        q = gco.view(np.int8).astype(np.int64) if bo == 8 else \
            np.stack([(gco & 0xF).astype(np.int64), (gco >> 4).astype(np.int64)], 1).reshape(-1)
        if bo == 4:
            q = np.where(q >= 8, q - 16, q)
        assert q[:4].tolist() == c["out_codes"], c["name"]


def test_empty_is_a_no_op():
    import block_quantization_codec_amd as z
    # numel == 0 with a requested output is valid and launches nothing
    g = Guarded(64)
    z.zpp_dequant_reduce_requant(g.ptr, 0, g.ptr, 0, 4, 4, 0, 256, None, None, 0, g.ptr)
    torch.cuda.synchronize()
    assert g.all_canary()


@pytest.mark.parametrize("bits_in,bits_out,R,block", [(4, 4, 8, 256), (8, 8, 3, 256), (4, 0, 5, 256),
                                                       (8, 4, 9, 256), (4, 8, 17, 256), (8, 0, 16, 256),
                                                       (4, 4, 8, 32), (8, 8, 5, 32), (4, 4, 8, 4096),
                                                       (8, 0, 3, 4096), (4, 4, 16, 256), (4, 0, 9, 128),
                                                       (4, 4, 1, 512)])
def test_wide_lane_path(bits_in, bits_out, R, block):
    """Outputs large enough for the 32-elements-per-lane layout (at least 4096 waves of
    2048 elements), with a ragged tail; the small cases above use 8 elements per lane.
    That layout sums batches of 8 inputs: fewer than 8, 9 and 17 inputs end in a
    partial batch, 8 and 16 do not; mixed code widths use their own kernels. With
    4-bit inputs and blocks up to 2048 the code vectors land in LDS slots: 16 inputs
    refill the slots once, 9 leave one live input in the second batch, 1 is a single
    input. Block 32 gives each lane a block of its own (no cross-lane maximum); block
    4096 spans two 2048-element segments per tile."""
    numel = 8192 * 2048 + (3 * 2048 + 5 * block if block < 2048 else 3 * block)   # a multiple of the block
    rng = np.random.default_rng([R, bits_in])
    per_c = numel * bits_in // 8
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    scales = np.exp2(rng.uniform(-20, -5, R * (numel // block))).astype(np.float32)
    gco, gso, gsu = _run(codes, per_c, scales, numel // block, R, bits_in, numel, block, bits_out)
    cl = [codes[r * per_c:(r + 1) * per_c] for r in range(R)]
    sl = [scales[r * (numel // block):(r + 1) * (numel // block)] for r in range(R)]
    co, so, su = oracle.dequant_reduce_requant(cl, sl, bits_in, numel, block, bits_out)
    assert_bits_equal(gsu, su, "sum (wide lanes)")
    if bits_out:
        assert_bits_equal(gso, so, "scales (wide lanes)")
        assert_bits_equal(gco, co, "codes (wide lanes)")


@pytest.mark.parametrize("R,bits_in,bits_out,waves", [(4, 4, 4, 1536), (4, 4, 4, 1535), (2, 4, 0, 1900),
                                                       (1, 4, 4, 1600), (5, 4, 4, 1600), (4, 8, 8, 1600),
                                                       (3, 4, 8, 2047)])
def test_layout_choice_for_few_inputs(R, bits_in, bits_out, waves):
    """With 4-bit codes and at most 4 inputs the 32-elements-per-lane layout
    is taken from 1,536 waves of 2,048 elements on (below that, and with 5
    inputs or 8-bit codes, the 8-element lanes up to 4,096 waves). Both sides
    of that choice, each with a ragged last tile, against the oracle."""
    block = 128
    numel = (waves - 1) * 2048 + 7 * block
    rng = np.random.default_rng([R, bits_in, waves])
    per_c = numel * bits_in // 8
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    scales = np.exp2(rng.uniform(-20, -5, R * (numel // block))).astype(np.float32)
    gco, gso, gsu = _run(codes, per_c, scales, numel // block, R, bits_in, numel, block, bits_out)
    cl = [codes[r * per_c:(r + 1) * per_c] for r in range(R)]
    sl = [scales[r * (numel // block):(r + 1) * (numel // block)] for r in range(R)]
    co, so, su = oracle_par.dequant_reduce_requant(cl, sl, bits_in, numel, block, bits_out)
    what = f"R={R} bits={bits_in}->{bits_out} waves={waves}"
    assert_bits_equal(gsu, su, "sum " + what)
    if bits_out:
        assert_bits_equal(gso, so, "scales " + what)
        assert_bits_equal(gco, co, "codes " + what)


# --------------------------------------------------------------------------
# zpp_dequant_reduce_average: the hop-2 sum divided by the GPU count
# --------------------------------------------------------------------------

def _run_avg(codes_np, cstride, scales_np, sstride, R, bits_in, numel, block, divisor):
    import block_quantization_codec_amd as z
    ci = dev(codes_np)
    si = dev(scales_np)
    ga = Guarded(4 * numel)
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_average(ci, cstride, si, sstride, R, bits_in, numel, block, divisor, ga.ptr)
    torch.cuda.synchronize()
    assert ga.untouched(), "write outside the output buffer"
    return ga.as_np(np.float32)


def _expect_avg(codes, per_c, scales, per_s, R, bits_in, numel, block, divisor):
    cl = [codes[r * per_c:r * per_c + numel * bits_in // 8] for r in range(R)]
    sl = [scales[r * per_s:r * per_s + numel // block] for r in range(R)]
    return oracle.dequant_average(cl, sl, bits_in, numel, block, divisor)


@pytest.mark.parametrize("divisor", [1, 3, 8, 24, 255, 256, 1000, 1 << 24])
@pytest.mark.parametrize("R,bits_in", [(1, 4), (5, 4), (32, 4), (3, 8), (9, 8)])
def test_average_matches_oracle(divisor, R, bits_in):
    block = 256
    numel = 37 * block  # several tiles and a ragged tail
    codes, pc, scales, ps = _inputs(R, bits_in, numel, block, 50 + divisor)
    got = _run_avg(codes, pc, scales, ps, R, bits_in, numel, block, divisor)
    want = _expect_avg(codes, pc, scales, ps, R, bits_in, numel, block, divisor)
    assert_bits_equal(got, want, f"average R={R} bits={bits_in} divisor={divisor}")


@pytest.mark.parametrize("block", BLOCKS)
def test_average_block_sizes(block):
    numel = 3 * 4096 + 2 * block
    codes, pc, scales, ps = _inputs(6, 4, numel, block, 7, gap=2)
    got = _run_avg(codes, pc, scales, ps, 6, 4, numel, block, 48)
    want = _expect_avg(codes, pc, scales, ps, 6, 4, numel, block, 48)
    assert_bits_equal(got, want, f"average block={block} (strided inputs)")


def test_average_wide_lane_path_and_power_of_two():
    """Large enough for 32 elements per lane; a power-of-two divisor equals the
    plain sum scaled exactly."""
    block, R = 256, 4
    numel = 8192 * 2048 + 7 * block
    rng = np.random.default_rng([91, R])
    per_c = numel // 2
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    scales = np.exp2(rng.uniform(-20, -5, R * (numel // block))).astype(np.float32)
    got = _run_avg(codes, per_c, scales, numel // block, R, 4, numel, block, 3)
    want = _expect_avg(codes, per_c, scales, numel // block, R, 4, numel, block, 3)
    assert_bits_equal(got, want, "average (wide lanes), divisor 3")
    got8 = _run_avg(codes, per_c, scales, numel // block, R, 4, numel, block, 8)
    _, _, total = _run(codes, per_c, scales, numel // block, R, 4, numel, block, 0)
    assert_bits_equal(got8, total * np.float32(0.125), "divisor 8 == sum / 8 exactly")


def test_golden_average_cases_on_gpu():
    """Hand-derived cases (blocks of 4) padded with zero codes to a block of 32."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "average_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        bi, R = c["bits"], len(c["inputs"])
        codes = np.zeros(R * 32 * bi // 8, np.uint8)
        scales = np.zeros(R, np.float32)
        for r, inp in enumerate(c["inputs"]):
            q = np.zeros(32, np.int64)
            q[:4] = inp["codes"]
            codes[r * 32 * bi // 8:(r + 1) * 32 * bi // 8] = _pack(q, bi)
            scales[r] = inp["scales"][0]
        got = _run_avg(codes, 32 * bi // 8, scales, 1, R, bi, 32, 32, c["divisor"])
        if "avg_bits_hex" in c:
            want = [int(h, 16) for h in c["avg_bits_hex"]]
            assert got[:4].view(np.uint32).tolist() == want, c["name"]
        else:
            assert got[:4].tolist() == c["avg"], c["name"]
        assert not got[4:].any()


def test_average_empty_is_a_no_op():
    import block_quantization_codec_amd as z
    g = Guarded(64)
    z.zpp_dequant_reduce_average(g.ptr, 0, g.ptr, 0, 4, 4, 0, 256, 3, g.ptr)
    torch.cuda.synchronize()
    assert g.all_canary()


@pytest.mark.parametrize("bits_in", [4, 8])
@pytest.mark.parametrize("R", [1, 2, 9, 17])
def test_zero_and_negative_scales_with_negative_codes(bits_in, R):
    """Negative codes with zero (or negative) scales give -0 products. The sum
    starts from +0 and adds every product, so where all products of an element
    are -0 the result is +0 (+0 + -0 = +0), and the requantized block is all
    zero. Arbitrary code bytes and scales are accepted by the entry point."""
    block = 64
    numel = 40 * block
    per_c = numel * bits_in // 8
    rng = np.random.default_rng([77, bits_in, R])
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    nb = numel // block
    scales = np.exp2(rng.uniform(-20, -5, R * nb)).astype(np.float32)
    scales[rng.random(R * nb) < 0.5] = 0.0          # zero scales in about half the blocks
    scales[rng.random(R * nb) < 0.1] *= -1.0        # and a few negative ones
    scales[:nb] = np.where(np.arange(nb) % 3 == 0, np.float32(0.0), scales[:nb])
    for bits_out in (0, 4, 8):
        gco, gso, gsu = _run(codes, per_c, scales, nb, R, bits_in, numel, block, bits_out)
        cl = [codes[r * per_c:(r + 1) * per_c] for r in range(R)]
        sl = [scales[r * nb:(r + 1) * nb] for r in range(R)]
        co, so, su = oracle.dequant_reduce_requant(cl, sl, bits_in, numel, block, bits_out)
        assert_bits_equal(gsu, su, f"sum with zero/negative scales, bits_out={bits_out}")
        if bits_out:
            assert_bits_equal(gso, so, "requantized scales")
            assert_bits_equal(gco, co, "requantized codes")
    avg = _run_avg(codes, per_c, scales, nb, R, bits_in, numel, block, 3)
    assert_bits_equal(avg, oracle.dequant_average(cl, sl, bits_in, numel, block, 3), "average")


@pytest.mark.parametrize("numel", [96 * 256, 4096 * 2048 + 7 * 256])
@pytest.mark.parametrize("R", [3, 8])
@pytest.mark.parametrize("bits_in", [4, 8])
def test_scales_on_both_sides_of_the_product_shortcut_bound(numel, R, bits_in):
    """Products are formed by a shortcut that is exact only for scales of
    magnitude at most 2^103 (4-bit codes) or 2^120 (8-bit codes); larger
    ones take the plain product. Blocks mix scales just inside and outside
    that bound with tiny (down to the smallest subnormal), zero and negative
    scales and arbitrary codes, on the 8- and 32-elements-per-lane layouts
    (the second size makes at least 4096 waves of 2048 elements). Only input
    0 gets scales near the bound and above it, and those stay at most
    1.5 * 2^124, so that every sum stays finite."""
    block = 256
    nb = numel // block
    per_c = numel * bits_in // 8
    rng = np.random.default_rng([119, R, numel, bits_in])
    codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
    f32 = np.float32
    top = f32(2.0 ** 103) if bits_in == 4 else f32(2.0 ** 120)
    far = f32(2.0 ** 124) if bits_in == 4 else f32(1.25 * 2.0 ** 120)   # well above the bound, sums finite
    big = np.array([top, np.nextafter(top, f32(np.inf)), -top, 1.5 * top, far, 0.75, 0.0], f32)
    small = np.array([2.0 ** 90, -(2.0 ** 100), 2.0 ** -122, np.nextafter(f32(2.0 ** -122), f32(0)),
                      -(2.0 ** -122), 3.0 * 2.0 ** -140, 2.0 ** -149, 2.0 ** -126, 0.0, -0.0, 0.75, -1e-3], f32)
    scales = rng.choice(small, R * nb).astype(f32)
    scales[:nb] = rng.choice(big, nb)
    scales[: nb // 4] = top                              # runs of blocks right at both ends
    scales[nb + nb // 4: nb + nb // 2] = f32(2.0 ** -122)
    cl = [codes[r * per_c:(r + 1) * per_c] for r in range(R)]
    sl = [scales[r * nb:(r + 1) * nb] for r in range(R)]
    for bits_out in (0, bits_in):
        gco, gso, gsu = _run(codes, per_c, scales, nb, R, bits_in, numel, block, bits_out)
        co, so, su = oracle.dequant_reduce_requant(cl, sl, bits_in, numel, block, bits_out)
        assert np.isfinite(su).all()
        assert_bits_equal(gsu, su, f"sum across the shortcut bound R={R} n={numel} bits={bits_in}")
        if bits_out:
            assert_bits_equal(gso, so, "requantized scales")
            assert_bits_equal(gco, co, "requantized codes")
    avg = _run_avg(codes, per_c, scales, nb, R, bits_in, numel, block, 7)
    assert_bits_equal(avg, oracle.dequant_average(cl, sl, bits_in, numel, block, 7), "average")
