"""The block-range thread pool gives the same bytes as one oracle call.

The GPU parity tests at the 500M-element and 855M-element sizes compare
against the oracle run in pieces (tests/oracle_par.py); this pins that the
pieces, concatenated, are byte-identical to a single call, for ragged block
counts and more pieces than blocks.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle_par
import synth


@pytest.mark.parametrize("block,bits,nblocks,threads", [(128, 4, 1001, 7), (512, 8, 37, 16), (32, 4, 3, 8),
                                                        (4096, 8, 5, 2), (256, 4, 1, 4)])
def test_quantize_and_dequantize_pieces_equal_one_call(block, bits, nblocks, threads):
    x = synth.small_bf16(block * nblocks, (0, 77, block, bits), 0.01, 1e-3, 100.0)
    c1, s1 = oracle.quantize(x, block, bits)
    c2, s2 = oracle_par.quantize(x, block, bits, n_threads=threads)
    assert c1.tobytes() == c2.tobytes() and s1.tobytes() == s2.tobytes()
    for out in ("f32", "bf16"):
        y1 = oracle.dequantize(c1, s1, bits, x.size, block, out=out)
        y2 = oracle_par.dequantize(c1, s1, bits, x.size, block, out=out, n_threads=threads)
        assert y1.tobytes() == y2.tobytes()


@pytest.mark.parametrize("bits_in,bits_out,n_inputs,block,nblocks", [(4, 4, 8, 256, 523), (4, 0, 32, 256, 61),
                                                                     (8, 8, 3, 64, 129), (8, 4, 5, 2048, 4)])
def test_hop_pieces_equal_one_call(bits_in, bits_out, n_inputs, block, nblocks):
    n = block * nblocks
    ins = [oracle.quantize(synth.small_bf16(n, (0, 78, r, block), 1e-3), block, bits_in) for r in range(n_inputs)]
    cs, ss = [i[0] for i in ins], [i[1] for i in ins]
    want = oracle.dequant_reduce_requant(cs, ss, bits_in, n, block, bits_out)
    got = oracle_par.dequant_reduce_requant(cs, ss, bits_in, n, block, bits_out, n_threads=6)
    for w, g in zip(want, got):
        assert (w is None) == (g is None)
        if w is not None:
            assert w.tobytes() == g.tobytes()
