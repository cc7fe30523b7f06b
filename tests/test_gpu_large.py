"""GPU parity beyond 2^31 elements (byte offsets beyond 2^32): 64-bit indexing.

One bf16 tensor of 517 * 2^22 = 2,168,455,168 elements (4.3 GB) goes through
every entry point. The input is a seeded pattern of 2^22 values, scaled in
each 2^22-element tile by its own power of two, so a 32-bit wrap of an index
or byte offset would read or write visibly different data. Outputs are
compared with the oracle on sampled blocks (the first and last blocks, the
blocks around element 2^31 and around every multiple of 2^29, where the hop
reduction starts another launch, and random ones); blocks are independent, so
the oracle recomputes exactly those from the same input values.

Two more tests go past the largest grid one launch can have (2^32 - 1
work-items, 16,777,215 workgroups of 256): dequantize past 2^35 elements (a
32 GiB int8 input, 64 GiB of bf16 out) and the bf16 4-bit quantize past 2^36
(128 GiB in), where waves take a second tile in their grid-stride loops. They
check the blocks on both sides of the first tile no first-pass wave covers.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_bits_equal, host, need_gpu, torch

pytestmark = pytest.mark.gpu

M = 1 << 22            # pattern length (elements)
TILES = 517            # tiles of M elements
N = TILES * M          # 2,168,455,168 > 2^31
EDGE = 1 << 31         # first element whose bf16 byte offset needs 33 bits
CHUNK = 1 << 29        # the hop kernels launch once per this many elements


@pytest.fixture(scope="module")
def x():
    need_gpu()
    pat = torch.from_numpy(synth.small_bf16(M, (0, 311), 0.02, 1e-3, 50.0)).view(torch.int16)
    pat = pat.view(torch.bfloat16).cuda().float()
    t = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    tv = t.view(TILES, M)
    for k in range(TILES):  # power-of-two tile scales: exact in bf16
        tv[k].copy_((pat * float(2.0 ** ((k % 61) - 30))).to(torch.bfloat16))
    torch.cuda.synchronize()
    yield t
    del t
    torch.cuda.empty_cache()


def _sample_blocks(block: int, seed: int) -> np.ndarray:
    nb = N // block
    rng = np.random.default_rng([seed, block])
    edges = [EDGE // block] + [k * CHUNK // block for k in range(1, N // CHUNK + 1)]
    idx = np.concatenate([np.arange(16), np.arange(nb - 16, nb), *[np.arange(e - 16, e + 16) for e in edges],
                          rng.choice(nb, 2000, replace=False)])
    return np.unique(idx)


def _gather_rows(t, width: int, idx: np.ndarray) -> np.ndarray:
    rows = t.view(-1, width)[torch.from_numpy(idx).cuda()]
    return host(rows).reshape(-1)


@pytest.mark.parametrize("bits,block", [(8, 256), (4, 128)])
def test_quantize_and_dequantize_past_2_31(x, bits, block):
    import block_quantization_codec_amd as z
    codes, scales = z.quantize(x, block, bits)
    y = z.dequantize(codes, scales, bits, N, block, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = _sample_blocks(block, bits)
    xs = _gather_rows(x, block, idx)
    oc, os_ = oracle.quantize(xs, block, bits)
    assert_bits_equal(_gather_rows(codes, block * bits // 8, idx), oc, f"int{bits} codes")
    assert_bits_equal(host(scales)[idx], os_, f"int{bits} scales")
    oy = oracle.dequantize(oc, os_, bits, xs.size, block, out="bf16")
    assert_bits_equal(_gather_rows(y, block, idx), oy, f"int{bits} dequantized bf16")
    del y
    # binary32 out: 8.7 GB, byte offsets past 2^33 (read back with slice copies)
    yf = z.dequantize(codes, scales, bits, N, block, dtype=torch.float32)
    torch.cuda.synchronize()
    of = oracle.dequantize(oc, os_, bits, xs.size, block, out="f32")
    assert_bits_equal(_rows_by_copies(yf, block, idx), of, f"int{bits} dequantized binary32")
    del codes, scales, yf


def test_reorder_and_fused_quantize_past_2_31(x):
    import block_quantization_codec_amd as z
    n, g, block = 2, 2, 256
    S = N // 4
    perm = oracle.reorder_permutation(n, g)
    out = z.reorder(x, n, g)
    fc, fs = z.quantize_reordered(x, n, g, block, 4)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    pos = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N), np.arange(EDGE - 64, EDGE + 64),
                                    rng.integers(0, N, 4000)]))
    src = np.asarray(perm, dtype=np.int64)[pos // S] * S + pos % S
    got = host(out[torch.from_numpy(pos).cuda()])
    want = host(x[torch.from_numpy(src).cuda()])
    assert_bits_equal(got, want, "reordered elements")
    del out
    idx = _sample_blocks(block, 9)
    blocks_per_slice = S // block
    src_blk = np.asarray(perm, dtype=np.int64)[idx // blocks_per_slice] * blocks_per_slice + idx % blocks_per_slice
    xs = _gather_rows(x, block, src_blk)
    oc, os_ = oracle.quantize(xs, block, 4)
    assert_bits_equal(_gather_rows(fc, block // 2, idx), oc, "fused reorder+quantize codes")
    assert_bits_equal(host(fs)[idx], os_, "fused reorder+quantize scales")
    del fc, fs


def test_hop_reduce_and_average_past_2_31(x):
    import block_quantization_codec_amd as z
    block, R = 128, 2
    cb, nb = N // 2, N // block
    codes = torch.empty(R * cb, dtype=torch.uint8, device="cuda")
    scales = torch.empty(R * nb, dtype=torch.float32, device="cuda")
    z.zpp_quantize_blocks(x, z.ZPP_BF16, N, block, 4, codes, scales)
    xr = torch.flip(x.view(TILES, M), [0]).reshape(-1)  # a second, different input
    z.zpp_quantize_blocks(xr, z.ZPP_BF16, N, block, 4, codes[cb:], scales[nb:])
    del xr
    co, so, su = z.dequant_reduce_requant(codes, scales, R, 4, N, block, bits_out=4, want_sum=True)
    avg = z.dequant_reduce_average(codes, scales, R, 4, N, block, 6)
    torch.cuda.synchronize()
    idx = _sample_blocks(block, 13)
    ci = [_gather_rows(codes[r * cb:(r + 1) * cb], block // 2, idx) for r in range(R)]
    si = [host(scales[r * nb:(r + 1) * nb])[idx] for r in range(R)]
    oco, oso, osu = oracle.dequant_reduce_requant(ci, si, 4, idx.size * block, block, 4)
    assert_bits_equal(_gather_rows(su, block, idx), osu, "hop sum")
    assert_bits_equal(_gather_rows(co, block // 2, idx), oco, "requantized codes")
    assert_bits_equal(host(so)[idx], oso, "requantized scales")
    oav = oracle.dequant_average(ci, si, 4, idx.size * block, block, 6)
    assert_bits_equal(_gather_rows(avg, block, idx), oav, "average over 6")
    del codes, scales, co, so, su, avg


GRID_WAVES = (0xFFFFFFFF // 256) * 4   # waves of the largest single-pass grid


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _need_device_bytes(n: int) -> None:
    """These tests hold tens of GiB at once; a device with less free memory
    skips them (with the figures) rather than failing the whole run."""
    _free()
    free, total = torch.cuda.mem_get_info()
    if free < n:
        pytest.skip(f"needs {n / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} of {total / 2**30:.0f} GiB free")


def _rows_by_copies(t, width: int, idx: np.ndarray) -> np.ndarray:
    """Rows idx of t viewed as [-1, width], read back with plain slice copies
    (runs of consecutive rows at a time). torch's index gather kernel faulted
    when it gathered rows of a 32 GiB tensor, so tensors this large are never
    indexed with an index tensor here."""
    idx = np.asarray(idx, dtype=np.int64)
    breaks = np.flatnonzero(np.diff(idx) != 1) + 1
    parts = []
    for run in np.split(idx, breaks):
        a, b = int(run[0]), int(run[-1]) + 1
        assert 0 <= a and b * width <= t.numel(), (a, b, width, t.numel())
        parts.append(host(t[a * width:b * width]))
    return np.concatenate(parts)


def _big_sample(nb: int, boundary_block: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([np.arange(16), np.arange(nb - 16, nb),
                                    np.arange(boundary_block - 32, boundary_block + 32),
                                    rng.choice(nb, 2000, replace=False)]))
    return idx[(idx >= 0) & (idx < nb)]


def test_dequantize_past_the_largest_grid():
    need_gpu()
    import block_quantization_codec_amd as z
    block = 256
    n = (1 << 35) + 5 * block                       # one-pass grid covers GRID_WAVES * 512 elements
    first_second_pass = GRID_WAVES * 512
    assert first_second_pass < n
    _need_device_bytes(n * 3 + (n // block) * 16 + (1 << 30))     # codes, bf16 out, scales and temporaries
    print(f"dequantize int8 -> bf16, {n} elements (tile {first_second_pass} starts the second pass)", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(41)
    codes = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
    e = torch.randint(-30, 31, (n // block,), device="cuda", generator=gen).float()
    scales = torch.exp2(e) * (1.0 + torch.rand(n // block, device="cuda", generator=gen))
    del e
    y = z.dequantize(codes, scales, 8, n, block, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = _big_sample(n // block, first_second_pass // block, 43)
    cs = _rows_by_copies(codes, block, idx)
    ss = _rows_by_copies(scales, 1, idx)
    want = oracle.dequantize(cs, ss, 8, idx.size * block, block, out="bf16")
    assert_bits_equal(_rows_by_copies(y, block, idx), want, "bf16 dequantized past the largest grid")
    del codes, scales, y
    _free()


def test_quantize_past_the_largest_grid():
    need_gpu()
    import block_quantization_codec_amd as z
    block = 128
    n = (1 << 36) + 3 * 1024                        # one-pass grid covers GRID_WAVES * 1024 elements
    first_second_pass = GRID_WAVES * 1024
    assert first_second_pass < n
    _need_device_bytes(n * 2 + n // 2 + (n // block) * 4 + (1 << 30))   # bf16 in, int4 codes, scales
    print(f"quantize bf16 -> int4, {n} elements (tile {first_second_pass} starts the second pass)", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(47)
    x = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    parts = 64
    step = (n + parts - 1) // parts
    for k in range(parts):  # normal values, a power-of-two scale per part
        x[k * step:(k + 1) * step].normal_(generator=gen).mul_(2.0 ** ((k % 9) - 4))
    codes, scales = z.quantize(x, block, 4)
    torch.cuda.synchronize()
    idx = _big_sample(n // block, first_second_pass // block, 53)
    xs = _rows_by_copies(x, block, idx)
    oc, os_ = oracle.quantize(xs, block, 4)
    assert_bits_equal(_rows_by_copies(codes, block // 2, idx), oc, "int4 codes past the largest grid")
    assert_bits_equal(_rows_by_copies(scales, 1, idx), os_, "int4 scales past the largest grid")
    del x, codes, scales
    _free()
