"""Host model of the qgZ two-hop exchange, used to pin the oracle's reorder.

Models the protocol of page "Quantized LLM Training at Scale with ZeRO++",
section "The Three Pillars of ZeRO++", pillar 3 (QGZ): every rank cuts its
(reordered) buffer into per-destination pieces, an intra-node all-to-all
delivers piece j to local rank j which reduces what it received, and an
inter-node all-to-all delivers sub-piece k of that result to node k, which
reduces again. The outcome it is checked against is the reduce-scatter of
page "ZeRO Stage 2: Gradient Partitioning": rank i ends with shard i
reduced over all ranks.

Ranks are node-major (rank = node * g + local). The model moves opaque
slice objects and combines them with a caller-supplied ``reduce``; it knows
nothing about the reorder's formula, which is passed in as a permutation.
"""
from __future__ import annotations

from collections import Counter
from typing import Callable, Sequence


def two_hop(buffers: Sequence[Sequence], n_nodes: int, g: int,
            permutation: Sequence[int] | None,
            reduce: Callable[[list], object]):
    """Run the two-hop exchange.

    ``buffers[r]`` is rank r's list of N = n_nodes * g slices in original
    order. ``permutation[p]`` is the original slice placed at position p
    before sending (``None``: no reorder). Returns ``(final, sent)`` where
    ``final[r]`` is what rank r holds after hop 2, and ``sent[r]`` counts the
    slices rank r sent in each hop as ``{"intra": x, "inter": y}``.
    """
    N = n_nodes * g
    assert all(len(b) == N for b in buffers)
    perm = list(range(N)) if permutation is None else list(permutation)
    assert sorted(perm) == list(range(N))
    staged = [[buffers[r][perm[p]] for p in range(N)] for r in range(N)]
    sent = [{"intra": 0, "inter": 0} for _ in range(N)]

    # hop 1: within node a, local rank i sends positions [j*n, (j+1)*n) to local j
    hop1 = [None] * N
    for a in range(n_nodes):
        for j in range(g):
            dst = a * g + j
            received = []
            for i in range(g):
                src = a * g + i
                piece = staged[src][j * n_nodes:(j + 1) * n_nodes]
                received.append(piece)
                if src != dst:
                    sent[src]["intra"] += len(piece)
            hop1[dst] = [reduce([received[i][k] for i in range(g)]) for k in range(n_nodes)]

    # hop 2: rank (a, j) sends sub-piece k of its hop-1 result to rank (k, j)
    final = [None] * N
    for k in range(n_nodes):
        for j in range(g):
            dst = k * g + j
            received = []
            for a in range(n_nodes):
                src = a * g + j
                received.append(hop1[src][k])
                if src != dst:
                    sent[src]["inter"] += 1
            final[dst] = reduce(received)
    return final, sent


def tagged_buffers(N: int):
    """Rank r's slice s is the multiset {(r, s)}."""
    return [[Counter({(r, s): 1}) for s in range(N)] for r in range(N)]


def multiset_union(items: list) -> Counter:
    out = Counter()
    for c in items:
        out.update(c)
    return out
