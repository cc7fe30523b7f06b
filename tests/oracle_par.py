"""The unchanged CPU oracle run over independent block ranges on a thread pool.

Blocks are independent in every routine the tests compare at full size
(quantize, dequantize, the hop reductions): each block's codes, scale and
sums depend only on that block's elements (page "Quantized LLM Training at
Scale with ZeRO++", section "The Three Pillars of ZeRO++": each chunk is
quantized on its own). So running the oracle on block-aligned pieces and
concatenating the pieces gives the same bytes as one call over everything,
which ``tests/test_oracle_par.py`` checks. The oracle's C routines run with
the GIL released (ctypes), so the pieces run in parallel.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _ranges(nblocks: int, parts: int):
    parts = max(1, min(parts, nblocks))
    step = -(-nblocks // parts)
    return [(b, min(nblocks, b + step)) for b in range(0, nblocks, step)]


def _run(fn, ranges, n_threads):
    if len(ranges) == 1:
        return [fn(*ranges[0])]
    with ThreadPoolExecutor(n_threads) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


def quantize(x: np.ndarray, block: int, bits: int, n_threads: int | None = None):
    """oracle.quantize over block ranges; returns (codes, scales)."""
    n_threads = n_threads or threads()
    nb = x.size // block

    def one(b0, b1):
        return oracle.quantize(x[b0 * block:b1 * block], block, bits)

    parts = _run(one, _ranges(nb, 4 * n_threads), n_threads)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def dequantize(codes: np.ndarray, scales: np.ndarray, bits: int, numel: int, block: int, out: str = "f32",
               n_threads: int | None = None) -> np.ndarray:
    n_threads = n_threads or threads()
    nb = numel // block
    cb = block * bits // 8

    def one(b0, b1):
        return oracle.dequantize(codes[b0 * cb:b1 * cb], scales[b0:b1], bits, (b1 - b0) * block, block, out=out)

    return np.concatenate(_run(one, _ranges(nb, 4 * n_threads), n_threads))


def dequant_reduce_requant(codes_list, scales_list, bits_in: int, numel: int, block: int, bits_out: int = 0,
                           n_threads: int | None = None):
    """oracle.dequant_reduce_requant over block ranges; returns (codes, scales, sum)."""
    n_threads = n_threads or threads()
    nb = numel // block
    cb = block * bits_in // 8

    def one(b0, b1):
        return oracle.dequant_reduce_requant([c[b0 * cb:b1 * cb] for c in codes_list],
                                             [s[b0:b1] for s in scales_list], bits_in, (b1 - b0) * block, block,
                                             bits_out)

    parts = _run(one, _ranges(nb, 4 * n_threads), n_threads)
    co = np.concatenate([p[0] for p in parts]) if bits_out else None
    so = np.concatenate([p[1] for p in parts]) if bits_out else None
    return co, so, np.concatenate([p[2] for p in parts])
