"""Exhaustive GPU check of the quantization rule over the whole bfloat16 domain.

For both code widths (Q = 127 and Q = 7) the production kernel behind
zpp_quantize_blocks sees every pair (x, a) of bfloat16 values with a a
positive finite block maximum and |x| <= a (both signs of x, -0 included):
about 1.07e9 pairs. Each block of 256 is [a, x_1 .. x_255], so its maximum
is exactly a, and its codes and scale must equal the oracle's bit for bit.
This covers every scale the codec can produce from bfloat16 input, including
subnormal ones, every rounding tie and every clamp; the GPU kernel's
division shortcut and scale split are thereby checked on the whole domain in
the production launch configuration.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gpu_util import assert_bits_equal, dev, need_gpu, torch

B = 256
PER_BLOCK = B - 1       # x values per block after the leading maximum a
A_MAX = 0x7F7F          # largest finite positive bfloat16
CHUNK_VALUES = 1 << 25  # x values per chunk (about 64 MiB of bf16 input)


def _chunks() -> list[tuple[int, int]]:
    """Ranges [a0, a1) of maxima whose value lists hold about CHUNK_VALUES."""
    out, a0, acc = [], 1, 0
    for a in range(1, A_MAX + 1):
        acc += 2 * a + 2
        if acc >= CHUNK_VALUES or a == A_MAX:
            out.append((a0, a + 1))
            a0, acc = a + 1, 0
    return out


def domain_blocks(a0: int, a1: int) -> np.ndarray:
    """Blocks [a, x...] for every maximum a in [a0, a1) and every x with |x| <= a.

    The x list of a is +0 .. +a, then -0 .. -a (bfloat16 bit patterns), laid
    PER_BLOCK to a block and padded with +0 (which leaves the maximum alone).
    """
    a = np.arange(a0, a1, dtype=np.int64)
    cnt = 2 * a + 2
    nb = -(-cnt // PER_BLOCK)
    first_row = np.concatenate(([0], np.cumsum(nb)[:-1]))
    out = np.zeros((int(nb.sum()), B), dtype=np.uint16)
    out[:, 0] = np.repeat(a, nb)
    owner = np.repeat(np.arange(a.size), cnt)
    i = np.arange(int(cnt.sum()), dtype=np.int64) - np.repeat(np.cumsum(cnt) - cnt, cnt)
    aa = a[owner]
    val = np.where(i <= aa, i, 0x8000 + (i - aa - 1))
    out[first_row[owner] + i // PER_BLOCK, 1 + i % PER_BLOCK] = val
    return out.reshape(-1)


def test_domain_generator_covers_every_pair():
    """The generator on a few maxima: each value list is exactly {x : |x| <= a}."""
    blocks = domain_blocks(1, 300).reshape(-1, B)
    for a in (1, 2, 254, 255, 256, 299):
        rows = blocks[blocks[:, 0] == a]
        assert rows.size
        xs = rows[:, 1:].reshape(-1)
        vals = np.sort(xs[: 2 * a + 2])
        want = np.sort(np.concatenate([np.arange(0, a + 1), 0x8000 + np.arange(0, a + 1)]).astype(np.uint16))
        assert np.array_equal(vals, want)
        assert np.all(xs[2 * a + 2:] == 0)  # padding
        mag = xs & 0x7FFF
        assert mag.max() == a


@pytest.mark.gpu
@pytest.mark.timeout(900)
def test_every_bf16_pair_matches_oracle():
    need_gpu()
    import block_quantization_codec_amd as z

    chunks = _chunks()
    workers = min(8, os.cpu_count() or 1)

    def prepare(rng):
        x = domain_blocks(*rng)
        return rng, x, oracle.quantize(x, B, 8), oracle.quantize(x, B, 4)

    def prepared():
        """Chunks in order, at most 2 * workers prepared ahead of the GPU."""
        with ThreadPoolExecutor(workers) as ex:
            pending = [ex.submit(prepare, c) for c in chunks[:2 * workers]]
            for k in range(len(chunks)):
                res = pending[k].result()
                pending[k] = None
                if k + 2 * workers < len(chunks):
                    pending.append(ex.submit(prepare, chunks[k + 2 * workers]))
                yield res

    pairs = 0
    for (a0, a1), x, (c8, s8), (c4, s4) in prepared():
        xd = dev(x)
        for bits, want_c, want_s in ((8, c8, s8), (4, c4, s4)):
            codes, scales = z.quantize(xd, B, bits)
            torch.cuda.synchronize()
            assert_bits_equal(codes.cpu().numpy(), want_c, f"int{bits} codes, maxima [{a0:#x}, {a1:#x})")
            assert_bits_equal(scales.cpu().numpy(), want_s, f"int{bits} scales, maxima [{a0:#x}, {a1:#x})")
        pairs += sum(2 * a + 2 for a in range(a0, a1))
        del xd
    assert pairs == sum(2 * a + 2 for a in range(1, A_MAX + 1))
    print(f"bf16 domain: {pairs} (x, a) pairs per code width match the oracle", flush=True)
