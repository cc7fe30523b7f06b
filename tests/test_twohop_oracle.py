"""The oracle's slice reorder and hop reductions against the two-hop protocol model.

Pins: the reorder must make the modelled two-hop exchange (page "Quantized
LLM Training at Scale with ZeRO++", section "The Three Pillars of ZeRO++",
QGZ) deliver exactly what a reduce-scatter delivers (page "ZeRO Stage 2:
Gradient Partitioning": GPU i ends with shard i, reduced over every GPU),
brute-forced for every grid of at most 8 ranks and checked index-only at
2x4 and 32x8. The numeric chain (reorder, one-shot 4-bit quantize, hop 1
with requantization, hop 2 sum) must land within the quantizers' error bound
of the exact sum, and must beat a ring reduce-scatter that requantizes at
every step (the precision loss the ZeRO++ page attributes to the ring).
"""
from __future__ import annotations

import json
import os
from collections import Counter

import numpy as np
import pytest

import oracle
import synth
from twohop_sim import multiset_union, tagged_buffers, two_hop

GRIDS = [(n, g) for n in range(1, 9) for g in range(1, 9) if n * g <= 8]


def _golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "reorder_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: f"{c['n_nodes']}x{c['gpus_per_node']}")
def test_golden_permutations(oracle_lib, case):
    assert oracle.reorder_permutation(case["n_nodes"], case["gpus_per_node"]) == case["src_of_position"]


@pytest.mark.parametrize("n,g", GRIDS)
def test_reorder_lands_every_slice_on_its_owner(oracle_lib, n, g):
    N = n * g
    perm = oracle.reorder_permutation(n, g)
    assert sorted(perm) == list(range(N))
    final, sent = two_hop(tagged_buffers(N), n, g, perm, multiset_union)
    for r in range(N):
        assert final[r] == Counter({(src, r): 1 for src in range(N)}), (n, g, r)
    for r in range(N):
        assert sent[r]["intra"] == (g - 1) * n
        assert sent[r]["inter"] == n - 1


@pytest.mark.parametrize("n,g", GRIDS)
def test_without_reorder_slices_are_misplaced(oracle_lib, n, g):
    N = n * g
    final, _ = two_hop(tagged_buffers(N), n, g, None, multiset_union)
    ok = all(final[r] == Counter({(src, r): 1 for src in range(N)}) for r in range(N))
    assert ok == (n == 1 or g == 1)
    if n == 1 or g == 1:
        assert oracle.reorder_permutation(n, g) == list(range(N))


@pytest.mark.parametrize("n,g", [(2, 4), (32, 8)])
def test_reorder_at_workload_grids(oracle_lib, n, g):
    N = n * g
    perm = oracle.reorder_permutation(n, g)
    final, _ = two_hop(tagged_buffers(N), n, g, perm, multiset_union)
    for r in range(N):
        assert final[r] == Counter({(src, r): 1 for src in range(N)})


@pytest.mark.parametrize("block", [128, 256])
@pytest.mark.parametrize("n,g", [(2, 4), (32, 8)])
def test_two_hop_send_volume_is_a_quarter(oracle_lib, n, g, block):
    """Per GPU, both hops together send less than 0.25 M (1 + 8/B) bytes of 4-bit
    codes plus scales, M being the bf16 bucket (the M -> 0.25M of QGZ)."""
    N = n * g
    _, sent = two_hop(tagged_buffers(N), n, g, oracle.reorder_permutation(n, g), multiset_union)
    slice_len = block * 64
    q_slice = slice_len // 2 + 4 * slice_len // block
    M = 2 * slice_len * N
    for r in range(N):
        total = (sent[r]["intra"] + sent[r]["inter"]) * q_slice
        assert total <= 0.25 * M * (1 + 8 / block)


def test_reorder_moves_bytes_of_any_width(oracle_lib):
    for slice_bytes in (1, 2, 3, 8, 16, 30_520):
        for n, g in [(2, 4), (4, 2), (3, 2)]:
            N = n * g
            buf = np.random.default_rng(slice_bytes).integers(0, 256, slice_bytes * N, dtype=np.uint8)
            out = oracle.reorder_slices(buf, n, g)
            perm = oracle.reorder_permutation(n, g)
            for p in range(N):
                s = perm[p]
                assert np.array_equal(out[p * slice_bytes:(p + 1) * slice_bytes],
                                      buf[s * slice_bytes:(s + 1) * slice_bytes])


# --------------------------------------------------------------------------
# numeric chain
# --------------------------------------------------------------------------

def _chain(bufs, n, g, block, slice_len):
    """Reorder, one-shot 4-bit quantize, hop 1 (dequant, sum, requant), hop 2 (dequant, sum)."""
    N = n * g
    chunk = slice_len * n
    qbufs = []
    for r in range(N):
        reordered = oracle.reorder_slices(bufs[r], n, g)
        qbufs.append(oracle.quantize(reordered, block, 4))
    hop1 = {}
    bound1 = {}
    for a in range(n):
        for j in range(g):
            cs = [qbufs[a * g + i][0][j * chunk // 2:(j + 1) * chunk // 2] for i in range(g)]
            ss = [qbufs[a * g + i][1][j * chunk // block:(j + 1) * chunk // block] for i in range(g)]
            co, so, _ = oracle.dequant_reduce_requant(cs, ss, 4, chunk, block, 4)
            hop1[a * g + j] = (co, so)
            bound1[a * g + j] = (np.sum([np.repeat(s.astype(np.float64), block) for s in ss], axis=0)
                                 * (0.5 + 2.0 ** -15) + np.repeat(so.astype(np.float64), block)
                                 * (0.5 + 2.0 ** -15))
    final, bound = {}, {}
    for k in range(n):
        for j in range(g):
            cs = [hop1[a * g + j][0][k * slice_len // 2:(k + 1) * slice_len // 2] for a in range(n)]
            ss = [hop1[a * g + j][1][k * slice_len // block:(k + 1) * slice_len // block] for a in range(n)]
            final[k * g + j] = oracle.dequant_sum(cs, ss, 4, slice_len, block)
            bound[k * g + j] = np.sum([bound1[a * g + j][k * slice_len:(k + 1) * slice_len]
                                       for a in range(n)], axis=0)
    return final, bound


@pytest.mark.parametrize("n,g", [(2, 4), (4, 2), (2, 2), (1, 4), (3, 2)])
def test_chain_reaches_reduce_scatter_within_bound(oracle_lib, n, g):
    N = n * g
    block = 128
    slice_len = block * 6
    bufs = [synth.small_bf16(slice_len * N, (21, n, g, r), 1e-3) for r in range(N)]
    final, bound = _chain(bufs, n, g, block, slice_len)
    vals = [oracle.bf16_decode(b).astype(np.float64) for b in bufs]
    for r in range(N):
        exact = np.sum([v[r * slice_len:(r + 1) * slice_len] for v in vals], axis=0)
        err = np.abs(final[r].astype(np.float64) - exact)
        slack = np.abs(exact) * 2.0 ** -20 + 1e-30
        assert np.all(err <= bound[r] + slack), (n, g, r, float(np.max(err - bound[r])))


def test_chain_is_exact_on_exactly_representable_data(oracle_lib):
    """Rank r holds c_r * base, where base has entries in {-1, 0, 1} and a 7 at
    the start of every block. Then every scale is an integer (7c/7), every
    code is base, every product and sum is a small integer: nothing rounds,
    and the chain must equal the reduce-scatter sum exactly."""
    n, g, block = 2, 4, 32
    N = n * g
    slice_len = block * 2
    rng = np.random.default_rng(8)
    base = rng.integers(-1, 2, slice_len * N).astype(np.float32)
    base[::block] = 7.0
    coef = rng.integers(1, 4, N).astype(np.float32)
    bufs = [oracle.bf16_round(base * coef[r]) for r in range(N)]
    final, _ = _chain(bufs, n, g, block, slice_len)
    for r in range(N):
        exact = base[r * slice_len:(r + 1) * slice_len].astype(np.float64) * coef.sum()
        assert np.array_equal(final[r].astype(np.float64), exact)


def _ring_reduce_scatter_requant(bufs, N, block, slice_len):
    """Ring reduce-scatter where each step dequantizes, adds its own slice and
    requantizes (4-bit) before passing on: N - 1 sequential requantizations."""
    out = {}
    for owner in range(N):
        start = (owner + 1) % N
        seg = oracle.bf16_decode(bufs[start][owner * slice_len:(owner + 1) * slice_len])
        c, s = oracle.quantize(seg, block, 4)
        for step in range(1, N):
            r = (start + step) % N
            mine = oracle.bf16_decode(bufs[r][owner * slice_len:(owner + 1) * slice_len])
            acc = (oracle.dequantize(c, s, 4, slice_len, block) + mine).astype(np.float32)
            if step < N - 1:
                c, s = oracle.quantize(acc, block, 4)
        out[owner] = acc
    return out


def test_one_shot_two_hop_beats_ring_requant(oracle_lib):
    n, g, block = 2, 4, 128
    N = n * g
    slice_len = block * 8
    bufs = [synth.small_bf16(slice_len * N, (31, r), 1e-3) for r in range(N)]
    final, _ = _chain(bufs, n, g, block, slice_len)
    ring = _ring_reduce_scatter_requant(bufs, N, block, slice_len)
    vals = [oracle.bf16_decode(b).astype(np.float64) for b in bufs]
    e2, er = [], []
    for r in range(N):
        exact = np.sum([v[r * slice_len:(r + 1) * slice_len] for v in vals], axis=0)
        e2.append(np.mean(np.abs(final[r] - exact)))
        er.append(np.mean(np.abs(ring[r] - exact)))
    print(f"mean abs error: two-hop {np.mean(e2):.3e}, ring with requant {np.mean(er):.3e}")
    assert np.mean(e2) < np.mean(er)
