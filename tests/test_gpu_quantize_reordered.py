"""GPU parity of zpp_quantize_reordered (slice reorder fused into the one-shot
quantize) against the oracle's quantize of the oracle's reorder.

Every output slice range, grid and block size must give exactly the codes and
scales that quantizing the reordered buffer gives for those slices (slices are
whole blocks, so the two steps commute with the range selection).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, assert_bits_equal, dev, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _run(x_np, slice_elems, n, g, first, count, block, bits):
    import block_quantization_codec_amd as z
    dt = z.ZPP_BF16 if x_np.dtype == np.uint16 else z.ZPP_FP32
    x = dev(x_np)
    out = slice_elems * count
    gc = Guarded(out * bits // 8)
    gs = Guarded(4 * (out // block))
    torch.cuda.synchronize()
    z.zpp_quantize_reordered(x, dt, slice_elems, n, g, first, count, block, bits, gc.ptr, gs.ptr)
    torch.cuda.synchronize()
    assert gc.untouched() and gs.untouched(), "write outside the output buffers"
    return gc.bytes(), gs.as_np(np.float32)


def _expect(x_np, slice_elems, n, g, first, count, block, bits):
    re_ = oracle.reorder_slices(x_np, n, g)
    part = re_[first * slice_elems:(first + count) * slice_elems]
    return oracle.quantize(part, block, bits)


def _input(N, slice_elems, f32, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(N * slice_elems).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, N * slice_elems // 32)).astype(np.float32).repeat(32)
    x[rng.choice(x.size, max(1, x.size // 500), replace=False)] *= 40
    return x if f32 else synth._f32_to_bf16_bits(x)


@pytest.mark.parametrize("n,g", [(2, 4), (4, 2), (3, 2), (1, 4), (8, 1), (32, 8)])
@pytest.mark.parametrize("bits,block", [(4, 256), (8, 512), (4, 128)])
def test_whole_buffer(n, g, bits, block):
    N = n * g
    slice_elems = block * (3 if N > 64 else 17)
    x = _input(N, slice_elems, False, (n, g, bits))
    got_c, got_s = _run(x, slice_elems, n, g, 0, N, block, bits)
    want_c, want_s = _expect(x, slice_elems, n, g, 0, N, block, bits)
    assert_bits_equal(got_s, want_s, "scales")
    assert_bits_equal(got_c, want_c, "codes")


@pytest.mark.parametrize("first,count", [(0, 1), (7, 1), (0, 7), (3, 4), (5, 3)])
def test_slice_ranges(first, count):
    n, g, block, bits = 2, 4, 256, 4
    slice_elems = block * 9
    x = _input(n * g, slice_elems, False, (first, count))
    got_c, got_s = _run(x, slice_elems, n, g, first, count, block, bits)
    want_c, want_s = _expect(x, slice_elems, n, g, first, count, block, bits)
    assert_bits_equal(got_s, want_s, "scales")
    assert_bits_equal(got_c, want_c, "codes")


@pytest.mark.parametrize("f32", [False, True], ids=["bf16", "f32"])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("block", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_block_sizes_and_types(block, bits, f32):
    n, g = 2, 2
    slice_elems = block * max(2, 6000 // block)   # several tiles, ragged against the tile size
    x = _input(n * g, slice_elems, f32, (block, bits, int(f32)))
    got_c, got_s = _run(x, slice_elems, n, g, 1, 3, block, bits)
    want_c, want_s = _expect(x, slice_elems, n, g, 1, 3, block, bits)
    assert_bits_equal(got_s, want_s, "scales")
    assert_bits_equal(got_c, want_c, "codes")


def test_empty_is_a_no_op():
    import block_quantization_codec_amd as z
    g = Guarded(64)
    z.zpp_quantize_reordered(g.ptr, z.ZPP_BF16, 256, 2, 4, 3, 0, 256, 4, g.ptr, g.ptr)
    torch.cuda.synchronize()
    assert g.all_canary()
