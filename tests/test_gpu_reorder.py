"""GPU parity of zpp_reorder_slices against the CPU oracle (bit-exact bytes).

Grids: every n_nodes x gpus_per_node with at most 8 ranks, plus 32x8 and a
64x2 grid; slice sizes that select every vector width (1, 2, 4, 8, 16 bytes)
and cover several tiles with a ragged tail; a 4-bit codes+scales pair laid
out like the 32x8 bucket's slices (976,640 code bytes and 30,520 scale bytes
per slice).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, assert_bits_equal, dev, need_gpu, torch

pytestmark = pytest.mark.gpu

GRIDS = [(n, g) for n in range(1, 9) for g in range(1, 9) if n * g <= 8] + [(32, 8), (64, 2)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _run(buf_np: np.ndarray, slice_bytes: int, n: int, g: int, in_offset: int = 0):
    import block_quantization_codec_amd as z
    src = dev(np.concatenate([np.zeros(in_offset, np.uint8), buf_np]))
    out = Guarded(buf_np.size)
    torch.cuda.synchronize()
    z.zpp_reorder_slices(src.data_ptr() + in_offset, out.ptr, slice_bytes, n, g)
    torch.cuda.synchronize()
    assert out.untouched(), "write outside the output buffer"
    return out.bytes()


@pytest.mark.parametrize("n,g", GRIDS)
@pytest.mark.parametrize("slice_bytes", [1, 2, 12, 24, 48, 16 * 4099, 30_520])
def test_reorder_matches_oracle(n, g, slice_bytes):
    if n * g > 64 and slice_bytes > 4096:
        slice_bytes = 4096 + 16
    N = n * g
    buf = np.random.default_rng([n, g, slice_bytes]).integers(0, 256, N * slice_bytes, dtype=np.uint8)
    got = _run(buf, slice_bytes, n, g)
    assert_bits_equal(got, oracle.reorder_slices(buf, n, g), f"reorder {n}x{g} slice={slice_bytes}")


@pytest.mark.parametrize("offset", [1, 2, 4, 8])
def test_unaligned_base_uses_narrower_vectors(offset):
    n, g, slice_bytes = 2, 4, 16 * 1000
    buf = np.random.default_rng(offset).integers(0, 256, n * g * slice_bytes, dtype=np.uint8)
    got = _run(buf, slice_bytes, n, g, in_offset=offset)
    assert_bits_equal(got, oracle.reorder_slices(buf, n, g), f"offset {offset}")


def test_reorder_of_codes_and_scales_at_32x8_slice_shape():
    """4-bit codes and scales of a bucket cut in 256 slices of 1,953,280 elements
    (7,630 blocks of 256): reordering them equals quantizing the reordered bf16
    (slices are whole blocks), checked on the oracle's outputs of a short bucket."""
    n, g, block = 32, 8, 256
    slice_elems = 256 * 16
    N = n * g
    x = np.random.default_rng(4).integers(0, 0x3F80, N * slice_elems).astype(np.uint16)
    codes, scales = oracle.quantize(x, block, 4)
    got_c = _run(codes, slice_elems // 2, n, g)
    got_s = _run(scales.view(np.uint8), 4 * slice_elems // block, n, g)
    rc, rs = oracle.quantize(oracle.reorder_slices(x, n, g), block, 4)
    assert_bits_equal(got_c, rc, "codes reorder == quantize(reorder)")
    assert_bits_equal(got_s.view(np.float32), rs, "scales reorder == quantize(reorder)")


def test_zero_slices_are_a_no_op():
    import block_quantization_codec_amd as z
    z.zpp_reorder_slices(None, None, 0, 2, 4)


def test_reorder_of_full_size_codes_and_scales_at_32x8():
    """The other unfused order of the 500M-element bucket at 32x8: its 4-bit
    codes (256 slices of 976,640 bytes) and scales (256 slices of 30,520 bytes,
    which take the 8-byte vector path) reordered as the benchmark does it,
    compared with the oracle's reorder in full."""
    n, g = 32, 8
    S = synth.QGZ_INT4_32x8.slice_len
    B = synth.QGZ_INT4_32x8.block
    N = n * g
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 256, N * S // 2, dtype=np.uint8)
    scales = rng.integers(0, 256, N * 4 * S // B, dtype=np.uint8)
    assert_bits_equal(_run(codes, S // 2, n, g), oracle.reorder_slices(codes, n, g), "codes at 32x8")
    assert_bits_equal(_run(scales, 4 * S // B, n, g), oracle.reorder_slices(scales, n, g), "scales at 32x8")
