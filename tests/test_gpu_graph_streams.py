"""The entry points under HIP graph capture and from several threads and streams.

The library keeps no per-call state and allocates nothing, so a sequence of
its calls can be captured once and replayed, and calls on different streams
can run at the same time. Graph test: the qgZ chain (reorder fused into the
4-bit quantize, hop 1 whole and split, hop 2 sum and average) and the 8-bit round trip are
captured into one graph, then replayed three times. Between replays the
program does its own eager work (it rewrites the inputs) and synchronizes,
and every replay must equal an eager run on the same inputs bit for bit.
Stream test: two host threads, each with its own stream, quantize different
tensors concurrently; every result equals the one-stream result.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

import synth
from gpu_util import assert_bits_equal, dev, host, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _z():
    import block_quantization_codec_amd as z
    return z


class Chain:
    """Buffers and launches of one small qgZ + qwZ sequence (2 nodes x 2 GPUs)."""

    def __init__(self):
        z = _z()
        self.n, self.g, self.B = 2, 2, 128
        n, g, B = self.n, self.g, self.B
        N = n * g
        self.S = 6 * B
        P = N * self.S
        self.P = P
        self.grad = dev(synth.small_bf16(P, (0, 401), 1e-3))
        self.w = dev(synth.small_bf16(64 * 256, (0, 402), 0.02, 1e-3, 50.0))
        self.qc = torch.empty(P // 2, dtype=torch.uint8, device="cuda")
        self.qs = torch.empty(P // B, dtype=torch.float32, device="cuda")
        C = n * self.S
        self.h1c = torch.empty(C // 2, dtype=torch.uint8, device="cuda")
        self.h1s = torch.empty(C // B, dtype=torch.float32, device="cuda")
        self.sc = torch.empty((C - self.S) // 2, dtype=torch.uint8, device="cuda")  # split hop 1: sent part
        self.ss = torch.empty((C - self.S) // B, dtype=torch.float32, device="cuda")
        self.kc = torch.empty(self.S // 2, dtype=torch.uint8, device="cuda")        # and kept sub-chunk 1
        self.ks = torch.empty(self.S // B, dtype=torch.float32, device="cuda")
        self.sum = torch.empty(self.S, dtype=torch.float32, device="cuda")
        self.avg = torch.empty(self.S, dtype=torch.float32, device="cuda")
        self.wc = torch.empty(self.w.numel(), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(self.w.numel() // 256, dtype=torch.float32, device="cuda")
        self.wy = torch.empty_like(self.w)
        self.z = z

    def launch(self):
        z, n, g, B, S = self.z, self.n, self.g, self.B, self.S
        C = n * S
        z.zpp_quantize_reordered(self.grad, z.ZPP_BF16, S, n, g, 0, n * g, B, 4, self.qc, self.qs)
        # hop 1 as local rank 0 of node 0 would run it: the g chunks 0 of the
        # reordered buffer stand in for the g local ranks' contributions
        z.zpp_dequant_reduce_requant(self.qc, 0, self.qs, 0, g, 4, C, B, self.h1c, self.h1s, 4, None)
        z.zpp_dequant_reduce_requant_split(self.qc, 0, self.qs, 0, g, 4, C, B, S, S, self.sc, self.ss, self.kc,
                                           self.ks, 4)
        z.zpp_dequant_reduce_requant(self.h1c, S // 2, self.h1s, S // B, n, 4, S, B, None, None, 0, self.sum)
        z.zpp_dequant_reduce_average(self.h1c, S // 2, self.h1s, S // B, n, 4, S, B, n * g, self.avg)
        z.zpp_quantize_blocks(self.w, z.ZPP_BF16, self.w.numel(), 256, 8, self.wc, self.ws)
        z.zpp_dequantize_blocks(self.wc, self.ws, 8, self.w.numel(), 256, self.wy, z.ZPP_BF16)

    def outputs(self):
        return [host(t).copy() for t in (self.qc, self.qs, self.h1c, self.h1s, self.sum, self.avg, self.wc,
                                         self.ws, self.wy, self.sc, self.ss, self.kc, self.ks)]

    def clear(self):
        for t in (self.qc, self.qs, self.h1c, self.h1s, self.sum, self.avg, self.wc, self.ws, self.wy, self.sc,
                  self.ss, self.kc, self.ks):
            t.view(torch.uint8).fill_(0xA5)


def test_graph_replays_equal_eager_runs():
    ch = Chain()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream, as torch recommends
        ch.launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ch.launch()
    torch.cuda.synchronize()
    names = ["codes", "scales", "hop-1 codes", "hop-1 scales", "hop-2 sum", "hop-2 average", "int8 codes",
             "int8 scales", "bf16 dequantized", "split hop-1 sent codes", "split hop-1 sent scales",
             "split hop-1 kept codes", "split hop-1 kept scales"]
    for rep, factor in enumerate((1.0, 2.0, 0.25)):
        if factor != 1.0:  # the program's own eager work between replays: new inputs
            ch.grad.mul_(factor)
            ch.w.mul_(-factor)
        torch.cuda.synchronize()
        ch.clear()
        ch.launch()
        torch.cuda.synchronize()
        eager = ch.outputs()
        ch.clear()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, ch.outputs(), eager):
            assert_bits_equal(got, want, f"replay {rep}: {name}")
    del graph


def test_threads_on_separate_streams():
    z = _z()
    xs = [dev(synth.small_bf16(1 << 20, (0, 410 + i), 0.02, 1e-3, 50.0)) for i in range(2)]
    ref = []
    for x in xs:
        c, s = z.quantize(x, 256, 8)
        ref.append((host(c), host(s)))
    torch.cuda.synchronize()
    outs = [[(torch.empty((1 << 20), dtype=torch.uint8, device="cuda"),
              torch.empty((1 << 20) // 256, dtype=torch.float32, device="cuda")) for _ in range(20)]
            for _ in range(2)]
    errors = []

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for c, s in outs[i]:
                    z.zpp_quantize_blocks(xs[i], z.ZPP_BF16, xs[i].numel(), 256, 8, c, s, st)
            st.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        for c, s in outs[i]:
            assert_bits_equal(host(c), ref[i][0], f"thread {i} codes")
            assert_bits_equal(host(s), ref[i][1], f"thread {i} scales")
    assert not np.array_equal(ref[0][0], ref[1][0])
