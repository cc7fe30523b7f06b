"""Pins of the host sizing module (block_quantization_codec_amd.plan).

Each value is pinned to a number the pages print, to an independent model of
the exchange (``twohop_sim.py``, which moves slices and counts what each rank
sends), or to properties that define the layout. Pages:
"Quantized LLM Training at Scale with ZeRO++" ("Understanding the ZeRO-3
Communication Volume": 3M per iteration for ZeRO-3, 0.75M for ZeRO++;
"The Three Pillars of ZeRO++": qwZ M -> 0.5M, hpZ M -> 0, qgZ M -> 0.25M);
"ZeRO-1/2/3" (16 bytes per parameter; 175B -> 2,800 GB, 7B -> 112 GB; the
stage formulas; stage 3 moves 1.5x the volume of plain data parallelism);
"ZeRO Stage 2: Gradient Partitioning" (the stage-2 memory equation and its
7B, N_d = 64 example).
"""
from __future__ import annotations

import pytest

import synth
from block_quantization_codec_amd import plan
from twohop_sim import two_hop

GB = 1e9


def test_zeropp_cuts_zero3_volume_from_3m_to_075m():
    v = plan.zeropp_volume()
    assert (v.forward_weights, v.backward_weights, v.gradients) == (0.5, 0.0, 0.25)
    assert v.total == 0.75 and v.zero3_total == 3.0 and v.reduction == 4.0


def test_block_scales_add_two_bytes_per_block_over_m():
    v = plan.zeropp_volume(weight_block=512, grad_block=256)
    assert v.forward_weights == 0.5 + 2 / 512
    assert v.gradients == 0.25 + 2 / 256
    assert plan.zeropp_volume(hpz=False).backward_weights == 1.0


def test_stage3_moves_one_and_a_half_times_data_parallel_volume():
    assert plan.zero_comm_volume(3) / plan.zero_comm_volume(0) == 1.5
    assert plan.zero_comm_volume(1) == plan.zero_comm_volume(2) == 2.0


def test_unsharded_memory_is_16_bytes_per_parameter():
    assert plan.zero_memory_per_gpu(175_000_000_000, 1, 0) == 2800 * GB
    assert plan.zero_memory_per_gpu(7_000_000_000, 64, 0) == 112 * GB


@pytest.mark.parametrize("stage", [0, 1, 2, 3])
def test_one_gpu_holds_everything_at_every_stage(stage):
    assert plan.zero_memory_per_gpu(1000, 1, stage) == 16_000


def test_stage_formulas():
    P, N = 7_000_000_000, 64
    assert plan.zero_memory_per_gpu(P, N, 1) == 4 * P + 12 * P / N
    assert plan.zero_memory_per_gpu(P, N, 3) == 16 * P / N
    s2 = plan.zero_memory_per_gpu(P, N, 2)
    assert s2 == 2 * P + 14 * P / N


def test_stage2_example_of_the_gradient_partitioning_page():
    """7B parameters on 64 GPUs: the replicated 16-bit parameters are 14 GB, as
    the page says. The page puts the sharded part at about 0.9 GB, but its own
    equation gives 14 * 7e9 / 64 = 1.53 GB (total 15.5 GB, not 14.9 GB); the
    module follows the equation, and the example stays unpinned beyond the
    14 GB term."""
    P, N = 7_000_000_000, 64
    assert 2 * P == 14 * GB
    s2 = plan.zero_memory_per_gpu(P, N, 2)
    assert s2 - 2 * P == pytest.approx(1.53125 * GB)
    assert s2 < 80 * GB  # fits one 80 GB accelerator, as the page concludes


@pytest.mark.parametrize("numel,n,g,block", [
    (500_000_000, 32, 8, 256), (16_000_000 * 8, 2, 4, 128), (1, 3, 5, 32), (0, 2, 2, 64), (4096, 2, 2, 1024)])
def test_slice_is_the_smallest_block_multiple_covering_the_bucket(numel, n, g, block):
    L = plan.qgz_layout(numel, n, g, block)
    N = n * g
    assert L.slice_elems % block == 0
    assert N * L.slice_elems >= numel
    assert L.slice_elems == 0 or N * (L.slice_elems - block) < numel
    assert L.padded_elems == N * L.slice_elems and L.chunk_elems == n * L.slice_elems
    assert sum(L.real_elems_of_rank(r) for r in range(N)) == numel


def test_layout_of_the_500m_bucket_at_32x8():
    L = plan.qgz_layout(500_000_000, 32, 8, 256)
    assert L.slice_elems == 1_953_280 and L.padded_elems == 500_039_680
    assert L.real_elems_of_rank(255) == 1_913_600
    c = synth.QGZ_INT4_32x8
    assert (c.slice_len, c.padded, c.chunk_len) == (L.slice_elems, L.padded_elems, L.chunk_elems)
    assert L.hop1_recv_bytes == 8 * (62_504_960 // 2 + 4 * 62_504_960 // 256)
    assert L.hop2_recv_bytes == 32 * (1_953_280 // 2 + 4 * 1_953_280 // 256)


@pytest.mark.parametrize("n,g", [(1, 2), (2, 1), (2, 2), (2, 3), (3, 2), (2, 4), (4, 2)])
def test_send_bytes_match_the_exchange_model(n, g):
    """The two-hop model counts the slices each rank sends in each hop."""
    L = plan.qgz_layout(10_000, n, g, 32)
    N = n * g
    _, sent = two_hop([[None] * N for _ in range(N)], n, g, list(range(N)), lambda xs: None)
    for r in range(N):
        assert sent[r]["intra"] * L.wire_bytes(L.slice_elems) == L.intra_node_send_bytes
        assert sent[r]["inter"] * L.wire_bytes(L.slice_elems) == L.inter_node_send_bytes


@pytest.mark.parametrize("block", [32, 256, 4096])
def test_per_gpu_send_volume_is_a_quarter_of_m_plus_scales(block):
    numel = 64 * 4096 * 32
    L = plan.qgz_layout(numel, 4, 8, block)
    M = 2 * numel
    sent = L.intra_node_send_bytes + L.inter_node_send_bytes
    assert sent <= 0.25 * M * (1 + 8 / block)
    assert sent == (L.n_ranks - 1) * L.wire_bytes(L.slice_elems)


def test_invalid_arguments():
    with pytest.raises(ValueError):
        plan.qgz_layout(100, 0, 2, 32)
    with pytest.raises(ValueError):
        plan.qgz_layout(100, 2, 2, 48)
    with pytest.raises(ValueError):
        plan.zero_memory_per_gpu(10, 0, 1)
    with pytest.raises(ValueError):
        plan.zero_comm_volume(4)
