"""Throughput of the ZeRO++ block-quantization codec on one MI355X.

One step is one pass of the whole per-GPU hot path on resident HBM inputs:

  qgZ, one GPU's share at 32 nodes x 8 GPUs (rank 255 = node 31, local 7),
  500,000,000-element bf16 gradient bucket (Student-t nu=3 x 1e-4),
  zero-padded to 256 slices of 1,953,280 elements, int4, block 256:
    1+2. tensor-slice reorder fused into the one-shot int4 quantize: the
       kernel reads the bucket in reordered slice order (chunks 0-6 of the
       reordered bucket into the send buffer, chunk 7 straight into its slot
       of the hop-1 receive buffer); the reordered bf16 bucket is never written
    3. hop 1: 8-way dequantize + fp32 sum + int4 requantize of the receive
       buffer in one launch (sub-chunks 0-30 into the hop-2 send buffer,
       sub-chunk 31 into its slot of the hop-2 receive buffer)
    4. hop 2: 32-way dequantize + fp32 sum into the owned fp32 shard
  qwZ and qgZ on one 70B-scale GQA layer (hidden 8192, 64/8 heads, FFN 28672,
  855,638,016 weights), N(0, 0.01) with 0.01 % outliers x100:
    5. int8 block-512 quantize of the bf16 weight
    6. dequantize of those codes back to bf16 (the gather side)
    7. int4 block-128 quantize of the bf16 gradient

The peers' hop-1 chunks and the other nodes' hop-2 pieces are drawn from the
same distributions and quantized once before timing (the exchanges are not
part of one GPU's work). Reported value: algorithmic input bytes of the six
kernel rows per step / step time (GB/s), the step timed over K back-to-back
steps with nothing between the kernels. The same K steps are then run again
with HIP events around every kernel row on the stream it runs on, and the
longest row is reported against the HBM roofline. Timed after the steps and
reported beside them: the unfused pair (standalone reorder of the bf16
bucket, then quantize of the reordered buffer), the other unfused order
(quantize the bucket as it is, then reorder its codes and scales), and hop 2
writing the averaged shard, a plain 1 GiB device copy (the slice reorder
with one slice) that each row is also compared with (`copy_frac`), for rows
moving less than 1 GiB a plain copy of the row's own read + write bytes with
its buffers rotated over 1 GiB (`of_copy_same_size`: how close the row comes
to what a copy of its size reaches, launch and ramp included), and the step
captured into a HIP graph and replayed (`graph_step`). The CPU baseline
runs the plain C oracle over the same work as one step (the reorder and the
quantize as two oracle steps), once on one core and twice on every core the
process may use (independent block ranges on a thread pool).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --configs       (one JSON line: kernel times at the 4096x4096,
       8 x 16M (2x4) and 64-shard shapes)
       python bench.py --block-sweep   (one JSON line: quantize / dequantize time
       and quantization error for every block size 32..4096, 8- and 4-bit codes,
       on the GQA weight, beside one global scale for the whole tensor)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

# source files each kernel family is built from (for the traffic record's validity)
KERNEL_SOURCES = {
    "quantize": ["quantize.hip", "zpp_device.h"],
    "dequantize": ["dequantize.hip", "zpp_device.h"],
    "reorder": ["reorder.hip", "zpp_device.h"],
    "drr": ["drr.hip", "drr_kernel.h", *(f"drr_in{i}_out{o}.hip" for i in (4, 8) for o in (0, 4, 8)),
            "zpp_device.h"],
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_hash(family: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "block_quantization_codec_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel_key: str, family: str):
    """Measured HBM bytes per launch from the committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(family):
        return None
    return rec.get("bytes_per_launch")


class Step:
    """Device buffers and the launch sequence of one step."""

    def __init__(self, torch, z, log_fn=log):
        import numpy as np

        import synth

        self.torch, self.z = torch, z
        dev = torch.device("cuda")
        c = synth.QGZ_INT4_32x8
        self.c = c
        n, g, B = c.n_nodes, c.gpus_per_node, c.block
        P, S, C = c.padded, c.slice_len, c.chunk_len
        self.node, self.local = n - 1, g - 1
        rank = self.node * g + self.local

        def to_dev(a):
            t = torch.from_numpy(a)
            if a.dtype == np.uint16:
                t = t.view(torch.int16).view(torch.bfloat16)
            return t.to(dev)

        t0 = time.time()
        log_fn(f"generating {c.name} rank {rank} ...")
        self.bucket_np = c.bucket(rank)
        self.bucket = to_dev(self.bucket_np)
        self.reord = torch.empty_like(self.bucket)
        # send / receive buffers (codes and scales) of the two hops
        self.send1_c = torch.empty((g - 1) * C // 2, dtype=torch.uint8, device=dev)
        self.send1_s = torch.empty((g - 1) * C // B, dtype=torch.float32, device=dev)
        self.recv1_c = torch.empty(g * C // 2, dtype=torch.uint8, device=dev)
        self.recv1_s = torch.empty(g * C // B, dtype=torch.float32, device=dev)
        self.send2_c = torch.empty((n - 1) * S // 2, dtype=torch.uint8, device=dev)
        self.send2_s = torch.empty((n - 1) * S // B, dtype=torch.float32, device=dev)
        self.recv2_c = torch.empty(n * S // 2, dtype=torch.uint8, device=dev)
        self.recv2_s = torch.empty(n * S // B, dtype=torch.float32, device=dev)
        self.shard = torch.empty(S, dtype=torch.float32, device=dev)
        self.avg_shard = torch.empty(S, dtype=torch.float32, device=dev)
        self.pre_c = torch.empty(P // 2, dtype=torch.uint8, device=dev)      # codes before the reorder
        self.pre_s = torch.empty(P // B, dtype=torch.float32, device=dev)
        self.post_c = torch.empty(P // 2, dtype=torch.uint8, device=dev)     # and after it
        self.post_s = torch.empty(P // B, dtype=torch.float32, device=dev)
        # what the exchanges would deliver: peers' chunks and other nodes' pieces
        for i in range(g - 1):
            x = to_dev(c.peer_chunk(i, self.local, self.node))
            z.zpp_quantize_blocks(x, z.ZPP_BF16, C, B, 4, self.recv1_c[i * C // 2:], self.recv1_s[i * C // B:])
        for a in range(n - 1):
            x = to_dev(c.node_partial(a, self.node, self.local))
            z.zpp_quantize_blocks(x, z.ZPP_FP32, S, B, 4, self.recv2_c[a * S // 2:], self.recv2_s[a * S // B:])
        torch.cuda.synchronize()
        log_fn(f"generating GQA layer weight and gradient ... ({time.time() - t0:.1f}s so far)")
        self.w_np = synth.gqa_weight()
        self.g_np = synth.gqa_grad()
        self.W = to_dev(self.w_np)
        self.G = to_dev(self.g_np)
        nw = self.W.numel()
        self.wc = torch.empty(nw, dtype=torch.uint8, device=dev)
        self.ws = torch.empty(nw // 512, dtype=torch.float32, device=dev)
        self.wy = torch.empty_like(self.W)
        self.gc = torch.empty(nw // 2, dtype=torch.uint8, device=dev)
        self.gs = torch.empty(nw // 128, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        log_fn(f"inputs resident in HBM ({time.time() - t0:.1f}s)")

        # (name, kernel family, algorithmic input bytes, algorithmic output bytes, rocprof name fragment)
        self.unfused_kernels = [
            ("reorder_bf16_256slices", "reorder", 2 * P, 2 * P, "reorder_kernel<16>"),
            ("quantize_int4_b256_of_reordered", "quantize", 2 * P, P // 2 + 4 * P // B,
             "quantize_kernel<4, 8, false> x2"),
        ]
        # beside the step: the optimizer-ready variant of hop 2 (sum averaged over
        # all n*g GPUs), and the other unfused order of rows a3/a4 (quantize the
        # bucket as it is, then reorder its codes and scales)
        self.extra_kernels = [
            ("hop2_average_256gpus_fp32", "drr", n * (S // 2 + 4 * S // B), 4 * S, "drr_kernel<4, 0, 8, 8> (avg)"),
            ("quantize_int4_b256_before_reorder", "quantize", 2 * P, P // 2 + 4 * P // B,
             "quantize_kernel<4, 8, false>"),
            ("reorder_int4_codes_and_scales", "reorder", P // 2 + 4 * P // B, P // 2 + 4 * P // B,
             "reorder_kernel<16> + reorder_kernel<8>"),
            ("hop1_two_launches_unsplit", "drr", g * (C // 2 + 4 * C // B), C // 2 + 4 * C // B,
             "drr_kernel<4, 4, 8, 32> + drr_kernel<4, 4, 8, 8>"),
        ]
        self.kernels = [
            ("reorder_quantize_int4_b256", "quantize", 2 * P, P // 2 + 4 * P // B,
             "quantize_kernel<4, 8, false> x2"),
            ("hop1_drr_8way_int4_b256", "drr", g * (C // 2 + 4 * C // B), C // 2 + 4 * C // B,
             "drr_kernel<4, 4, 8, 32>"),
            ("hop2_reduce_32way_fp32", "drr", n * (S // 2 + 4 * S // B), 4 * S, "drr_kernel<4, 0, 8, 8>"),
            ("quantize_int8_b512_gqa_weight", "quantize", 2 * nw, nw + 4 * nw // 512,
             "quantize_kernel<8, 9, false>"),
            ("dequantize_int8_b512_gqa_weight", "dequantize", nw + 4 * nw // 512, 2 * nw,
             "dequantize_kernel<8, false>"),
            ("quantize_int4_b128_gqa_grad", "quantize", 2 * nw, nw // 2 + 4 * nw // 128,
             "quantize_kernel<4, 7, false>"),
        ]

    def launches(self):
        """One step: a list of zero-argument callables, one per kernel row."""
        z, c = self.z, self.c
        n, g, B = c.n_nodes, c.gpus_per_node, c.block
        S, C = c.slice_len, c.chunk_len
        loc, node = self.local, self.node
        nw = self.W.numel()

        def reorder_quantize_grad():
            # slice reorder fused into the one-shot quantize: chunks 0..loc-1 of the
            # reordered bucket into the send buffer, chunk loc into its receive slot
            z.zpp_quantize_reordered(self.bucket, z.ZPP_BF16, S, n, g, 0, loc * n, B, 4, self.send1_c,
                                     self.send1_s)
            z.zpp_quantize_reordered(self.bucket, z.ZPP_BF16, S, n, g, loc * n, n, B, 4,
                                     self.recv1_c[loc * C // 2:], self.recv1_s[loc * C // B:])

        def hop1():
            # one pass: sub-chunk `node` (this GPU's own) straight into its slot of
            # the hop-2 receive buffer, the other 31 into the hop-2 send buffer
            z.zpp_dequant_reduce_requant_split(self.recv1_c, C // 2, self.recv1_s, C // B, g, 4, C, B, node * S, S,
                                               self.send2_c, self.send2_s, self.recv2_c[node * S // 2:],
                                               self.recv2_s[node * S // B:], 4)

        def hop2():
            z.zpp_dequant_reduce_requant(self.recv2_c, S // 2, self.recv2_s, S // B, n, 4, S, B, None, None, 0,
                                         self.shard)

        def qw():
            z.zpp_quantize_blocks(self.W, z.ZPP_BF16, nw, 512, 8, self.wc, self.ws)

        def dqw():
            z.zpp_dequantize_blocks(self.wc, self.ws, 8, nw, 512, self.wy, z.ZPP_BF16)

        def qg():
            z.zpp_quantize_blocks(self.G, z.ZPP_BF16, nw, 128, 4, self.gc, self.gs)

        return [reorder_quantize_grad, hop1, hop2, qw, dqw, qg]

    def unfused_launches(self):
        """The same qgZ first step unfused: the standalone slice reorder of the
        bf16 bucket, then the quantize of the reordered bucket."""
        z, c = self.z, self.c
        n, g, B = c.n_nodes, c.gpus_per_node, c.block
        S, C = c.slice_len, c.chunk_len
        loc = self.local

        def reorder():
            z.zpp_reorder_slices(self.bucket, self.reord, 2 * S, n, g)

        def quantize_reordered_buffer():
            z.zpp_quantize_blocks(self.reord, z.ZPP_BF16, loc * C, B, 4, self.send1_c, self.send1_s)
            z.zpp_quantize_blocks(self.reord[loc * C:], z.ZPP_BF16, C, B, 4, self.recv1_c[loc * C // 2:],
                                  self.recv1_s[loc * C // B:])

        return [reorder, quantize_reordered_buffer]


    def extra_launches(self):
        """Kernels reported beside the step: hop 2 writing the averaged shard."""
        z, c = self.z, self.c
        n, g, B = c.n_nodes, c.gpus_per_node, c.block
        S = c.slice_len

        def hop2_average():
            z.zpp_dequant_reduce_average(self.recv2_c, S // 2, self.recv2_s, S // B, n, 4, S, B, n * g,
                                         self.avg_shard)

        def quantize_before_reorder():
            z.zpp_quantize_blocks(self.bucket, z.ZPP_BF16, n * g * S, B, 4, self.pre_c, self.pre_s)

        def reorder_codes_and_scales():
            z.zpp_reorder_slices(self.pre_c, self.post_c, S // 2, n, g)
            z.zpp_reorder_slices(self.pre_s, self.post_s, 4 * S // B, n, g)

        def hop1_two_launches():
            # hop 1 as two calls of the unsplit step: sub-chunks 0..node-1 to the
            # send buffer, then sub-chunk `node` to its receive slot
            node = self.node
            C = c.chunk_len
            z.zpp_dequant_reduce_requant(self.recv1_c, C // 2, self.recv1_s, C // B, g, 4, node * S, B,
                                         self.send2_c, self.send2_s, 4, None)
            z.zpp_dequant_reduce_requant(self.recv1_c[node * S // 2:], C // 2, self.recv1_s[node * S // B:],
                                         C // B, g, 4, S, B, self.recv2_c[node * S // 2:],
                                         self.recv2_s[node * S // B:], 4, None)

        return [hop2_average, quantize_before_reorder, reorder_codes_and_scales, hop1_two_launches]


def time_rows(torch, stream, fns, table, K):
    """Average HIP-event time of each callable over K rounds, after one untimed round."""
    for f in fns:
        f()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(K)]
    for k in range(K):
        for i, f in enumerate(fns):
            ev[k][i][0].record(stream)
            f()
            ev[k][i][1].record(stream)
    torch.cuda.synchronize()
    out = {}
    for i, (name, _, rin, wout, _) in enumerate(table):
        ms = sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(K)) / K
        out[name] = {"ms": round(ms, 5),
                     "hbm_frac": round((rin + wout) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    return out


def graph_step_ms(torch, fns, K):
    """Milliseconds per step when the step's launches are captured into one HIP
    graph and the graph is replayed K times back to back."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager pass on the capture stream first
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for f in fns:
            f()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    del graph
    return ms


def copy_ceiling(torch, z, stream, K):
    """A plain device copy through the library's own slice reorder (one slice
    of 1 GiB: non-temporal 16-byte loads, streaming stores), timed with HIP
    events over K launches: the practical read + write rate the codec
    kernels are compared with beside the 8 TB/s peak."""
    n = 1 << 30
    src = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        z.zpp_reorder_slices(src, dst, n, 1, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        z.zpp_reorder_slices(src, dst, n, 1, 1)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / K
    del src, dst
    gbps = 2 * n / (ms * 1e-3) / 1e9
    return {"what": "zpp_reorder_slices over one 1 GiB slice (a plain copy)", "rocprof_name": "reorder_kernel<16>",
            "bytes": 2 * n, "ms": round(ms, 5), "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


_SAME_SIZE_COPY = {}


def same_size_copy(torch, z, stream, rw_bytes: int, K: int) -> float:
    """Mean HIP-event time (ms) of a plain device copy that reads and writes
    as many bytes as a row does (rw_bytes in total), through the library's
    one-slice reorder, with sources and destinations rotated over at least
    1 GiB so every launch reads from HBM: the rate a kernel of that size can
    reach, launch and ramp included, against which the small rows are read."""
    import math
    half = max(4096, (rw_bytes // 2 + 4095) // 4096 * 4096)
    if half in _SAME_SIZE_COPY:
        return _SAME_SIZE_COPY[half]
    ncopy = max(2, math.ceil(ROTATE_BYTES / (2 * half)))
    src = [torch.zeros(half, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    for k in range(ncopy):
        z.zpp_reorder_slices(src[k], dst[k], half, 1, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(ev):
        a.record(stream)
        z.zpp_reorder_slices(src[(k + 1) % ncopy], dst[(k + 1) % ncopy], half, 1, 1)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / K
    del src, dst
    _SAME_SIZE_COPY[half] = ms
    return ms


def _block_ranges(nblocks: int, parts: int):
    parts = max(1, min(parts, nblocks))
    step = -(-nblocks // parts)
    return [(b, min(nblocks, b + step)) for b in range(0, nblocks, step)]


def cpu_baseline(step: "Step", passes_one: int = 1, passes_all: int = 2):
    """The oracle, as it stands, over the same work as one step: once on one
    core, then on every core this process may use. The all-cores leg runs the
    unchanged oracle over independent pieces on a thread pool (ctypes releases
    the GIL during each oracle call): block ranges for the quantizers, the
    dequantizer and the hop reductions, and column ranges of the [slices]
    [slice] view for the reorder (each slice's columns move as a whole).
    Blocks and columns are independent, so the pieces are the same work. The
    reorder and the quantize are separate oracle steps (the oracle has no
    fused kernel)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    oracle.lib()
    c = step.c
    n, g, B = c.n_nodes, c.gpus_per_node, c.block
    N, S, Cl = n * g, c.slice_len, c.chunk_len
    nw = step.w_np.size
    bucket = step.bucket_np
    hc, hs = oracle.quantize(bucket[:Cl], B, 4)       # hop inputs (their values do not change the work)
    h2c, h2s = oracle.quantize(bucket[:S], B, 4)
    w_q = oracle.quantize(step.w_np, 512, 8)
    cores = len(os.sched_getaffinity(0))
    PARTS = 4 * cores
    # the reorder's pieces: column ranges of the [N][S] view, made contiguous beforehand
    cols = [(c0, c1) for c0, c1 in _block_ranges(S // B, PARTS)]
    re_pieces = [np.ascontiguousarray(bucket.reshape(N, S)[:, c0 * B:c1 * B]).reshape(-1) for c0, c1 in cols]
    reordered = oracle.reorder_slices(bucket, n, g)

    def work(pool):
        """(name, input bytes, callable) for every kernel row of one step."""
        def par(fn, nblocks):
            rs = _block_ranges(nblocks, PARTS if pool else 1)
            if pool is None:
                return lambda: [fn(*r) for r in rs]
            return lambda: list(pool.map(lambda r: fn(*r), rs))

        reorder = (lambda: oracle.reorder_slices(bucket, n, g)) if pool is None else \
            (lambda: list(pool.map(lambda i: oracle.reorder_slices(re_pieces[i], n, g), range(len(re_pieces)))))
        return [
            ("reorder", bucket.nbytes, reorder),
            ("quantize_int4_b256", reordered.nbytes,
             par(lambda b0, b1: oracle.quantize(reordered[b0 * B:b1 * B], B, 4), reordered.size // B)),
            ("hop1", g * (Cl // 2 + 4 * Cl // B),
             par(lambda b0, b1: oracle.dequant_reduce_requant([hc[b0 * B // 2:b1 * B // 2]] * g, [hs[b0:b1]] * g, 4,
                                                              (b1 - b0) * B, B, 4), Cl // B)),
            ("hop2", n * (S // 2 + 4 * S // B),
             par(lambda b0, b1: oracle.dequant_reduce_requant([h2c[b0 * B // 2:b1 * B // 2]] * n, [h2s[b0:b1]] * n,
                                                              4, (b1 - b0) * B, B, 0), S // B)),
            ("quantize_int8_b512", 2 * nw,
             par(lambda b0, b1: oracle.quantize(step.w_np[b0 * 512:b1 * 512], 512, 8), nw // 512)),
            ("dequantize_int8_b512", nw + 4 * nw // 512,
             par(lambda b0, b1: oracle.dequantize(w_q[0][b0 * 512:b1 * 512], w_q[1][b0:b1], 8, (b1 - b0) * 512, 512,
                                                  out="bf16"), nw // 512)),
            ("quantize_int4_b128", 2 * nw,
             par(lambda b0, b1: oracle.quantize(step.g_np[b0 * 128:b1 * 128], 128, 4), nw // 128)),
        ]

    def leg(pool, passes):
        timings = []
        for _ in range(passes):
            for name, nb, fn in work(pool):
                t = time.perf_counter()
                fn()
                timings.append((name, nb, time.perf_counter() - t))
        total_in = sum(t[1] for t in timings)
        total_s = sum(t[2] for t in timings)
        return {"GBps": round(total_in / total_s / 1e9, 4), "seconds": round(total_s, 2),
                "input_GB": round(total_in / 1e9, 2), "passes": passes,
                "per_kernel_s": {k: round(sum(t[2] for t in timings if t[0] == k), 3)
                                 for k in dict.fromkeys(t[0] for t in timings)}}

    one = leg(None, passes_one)
    with ThreadPoolExecutor(cores) as pool:
        allc = leg(pool, passes_all)
    return {
        "value": allc["GBps"],
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"all of every kernel's work in one step ({S}-element slices, {Cl}-element hop-1 chunk, "
                   f"{nw}-element GQA weight and gradient), {passes_all} passes on {cores} threads over "
                   f"independent block ranges ({allc['input_GB']} GB of input in {allc['seconds']} s); "
                   f"one_core: the same work, {passes_one} pass on one thread"),
        "seconds": allc["seconds"],
        "cpu_model": cpu_model(),
        "per_kernel_s": allc["per_kernel_s"],
        "one_core": {"value": one["GBps"], "unit": "GB/s", "cores": 1, "seconds": one["seconds"],
                     "per_kernel_s": one["per_kernel_s"]},
    }


ROTATE_BYTES = 1 << 30  # input and output copies a smaller-workload row cycles through


def configs_bench(torch, z, K: int = 50) -> dict:
    """Kernel times at the three smaller workload shapes (the 500M-element
    bucket and the GQA layer are the step's rows). Each row cycles through
    copies of its inputs and outputs totalling at least 1 GiB, so every launch
    reads inputs last touched a gigabyte of traffic earlier (out of the
    256 MB Infinity Cache) and writes outputs that are not resident either;
    each launch is timed with HIP events (mean, p10, p50, p90 over K
    launches, after one untimed pass over all copies)."""
    import math

    import numpy as np

    import synth

    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()

    def to_dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return t.view(torch.int16).view(torch.bfloat16).to(dev) if a.dtype == np.uint16 else t.to(dev)

    def nbytes(ts):
        return sum(t.numel() * t.element_size() for t in ts)

    def rows(table):
        """table: [(name, buffers, fn(buffers), read bytes, write bytes)] -> {name: timing}"""
        out = {}
        for name, bufs, fn, rb, wb in table:
            ncopy = max(2, math.ceil(ROTATE_BYTES / nbytes(bufs)))
            copies = [bufs] + [tuple(t.clone() for t in bufs) for _ in range(ncopy - 1)]
            for c in copies:
                fn(c)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
            torch.cuda.synchronize()
            for k, (a, b) in enumerate(ev):
                a.record(stream)
                fn(copies[(k + 1) % ncopy])
                b.record(stream)
            torch.cuda.synchronize()
            ts = sorted(a.elapsed_time(b) for a, b in ev)
            ms = sum(ts) / K
            del copies
            cms = same_size_copy(torch, z, stream, rb + wb, K)
            out[name] = {"ms": round(ms, 5), "ms_p10": round(ts[int(0.1 * (K - 1))], 5),
                         "ms_p50": round(ts[(K - 1) // 2], 5), "ms_p90": round(ts[int(0.9 * (K - 1) + 0.5)], 5),
                         "in_GBps": round(rb / (ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round((rb + wb) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "rw_bytes": rb + wb,
                         "copy_same_size_ms": round(cms, 5), "of_copy_same_size": round(cms / ms, 4),
                         "copies": ncopy, "rotated_bytes": ncopy * nbytes(bufs)}
            log(f"{name}: {ms * 1e3:.1f} us, {out[name]['hbm_frac']:.3f} of HBM peak, "
                f"{cms / ms:.3f} of a same-size copy ({ncopy} copies)")
        return out

    res = {}
    # 4096 x 4096 weight, int8 block 256: quantize and dequantize
    c1 = synth.QWZ_INT8_4096
    n1, B1 = c1.numel, c1.block
    x1 = to_dev(c1.weight())
    q1c = torch.empty(n1, dtype=torch.uint8, device=dev)
    q1s = torch.empty(n1 // B1, dtype=torch.float32, device=dev)
    z.zpp_quantize_blocks(x1, z.ZPP_BF16, n1, B1, 8, q1c, q1s)
    y1 = torch.empty_like(x1)
    res[c1.name] = rows([
        ("quantize_int8_b256", (x1, q1c, q1s),
         lambda b: z.zpp_quantize_blocks(b[0], z.ZPP_BF16, n1, B1, 8, b[1], b[2]), 2 * n1, n1 + 4 * n1 // B1),
        ("dequantize_int8_b256_bf16", (q1c, q1s, y1),
         lambda b: z.zpp_dequantize_blocks(b[0], b[1], 8, n1, B1, b[2], z.ZPP_BF16), n1 + 4 * n1 // B1, 2 * n1),
    ])
    del x1, q1c, q1s, y1
    # 8 ranks x 16M at 2 x 4, int4 block 128
    c2 = synth.QGZ_INT4_2x4
    n, g, N, B2 = c2.n_nodes, c2.gpus_per_node, c2.n_ranks, c2.block
    P, S, C = c2.padded, c2.slice_len, c2.chunk_len
    grads = to_dev(np.concatenate([c2.bucket(r) for r in range(N)]))
    reord = torch.empty_like(grads)
    q2c = torch.empty(N * P // 2, dtype=torch.uint8, device=dev)
    q2s = torch.empty(N * P // B2, dtype=torch.float32, device=dev)
    h2c = torch.empty(n * P // 2, dtype=torch.uint8, device=dev)
    h2s = torch.empty(n * P // B2, dtype=torch.float32, device=dev)
    for r in range(N):
        z.zpp_reorder_slices(grads[r * P:], reord[r * P:], 2 * S, n, g)
    z.zpp_quantize_blocks(reord, z.ZPP_BF16, N * P, B2, 4, q2c, q2s)
    torch.cuda.synchronize()
    a, j = n - 1, g - 1  # rank 7's share: chunk j of node a's local ranks
    one_off = a * g * P + j * C
    # one GPU's share as it would arrive: its 4 inputs side by side
    sh_c = q2c.view(N, P // 2)[a * g:(a + 1) * g, j * C // 2:(j + 1) * C // 2].contiguous().view(-1)
    sh_s = q2s.view(N, P // B2)[a * g:(a + 1) * g, j * C // B2:(j + 1) * C // B2].contiguous().view(-1)
    o1c = torch.empty(C // 2, dtype=torch.uint8, device=dev)
    o1s = torch.empty(C // B2, dtype=torch.float32, device=dev)
    del one_off

    def reorder_all(b):
        for r in range(N):
            z.zpp_reorder_slices(b[0][r * P:], b[1][r * P:], 2 * S, n, g)

    def hop1_all(b):
        for aa in range(n):
            z.zpp_dequant_reduce_requant(b[0][aa * g * P // 2:], P // 2, b[1][aa * g * P // B2:], P // B2, g, 4, P,
                                         B2, b[2][aa * P // 2:], b[3][aa * P // B2:], 4, None)

    w1 = g * (C // 2 + 4 * C // B2)
    res[c2.name] = rows([
        ("reorder_bf16_8_ranks", (grads, reord), reorder_all, 2 * N * P, 2 * N * P),
        ("quantize_int4_b128_8_ranks", (reord, q2c, q2s),
         lambda b: z.zpp_quantize_blocks(b[0], z.ZPP_BF16, N * P, B2, 4, b[1], b[2]),
         2 * N * P, N * P // 2 + 4 * N * P // B2),
        ("hop1_4way_one_share", (sh_c, sh_s, o1c, o1s),
         lambda b: z.zpp_dequant_reduce_requant(b[0], C // 2, b[1], C // B2, g, 4, C, B2, b[2], b[3], 4, None),
         w1, C // 2 + 4 * C // B2),
        ("hop1_4way_all_8_shares", (q2c, q2s, h2c, h2s), hop1_all, N * w1, N * (C // 2 + 4 * C // B2)),
    ])
    # hop 2 of the same grid for one GPU (node n-1, local rank g-1): its slice
    # of both nodes' hop-1 outputs (filled by the hop-1 row above), summed in
    # binary32
    off2 = (g - 1) * C + (n - 1) * S
    o2 = torch.empty(S, dtype=torch.float32, device=dev)
    res[c2.name].update(rows([
        ("hop2_2way_one_shard_fp32", (h2c, h2s, o2),
         lambda b: z.zpp_dequant_reduce_requant(b[0][off2 // 2:], P // 2, b[1][off2 // B2:], P // B2, n, 4, S, B2,
                                                None, None, 0, b[2]),
         n * (S // 2 + 4 * S // B2), 4 * S),
    ]))
    del grads, reord, q2c, q2s, h2c, h2s, sh_c, sh_s, o1c, o1s, o2
    # 64 int8 shards (block 2048) of a Llama-style layer, dequantized in one launch
    c3 = synth.QWZ_DEQUANT_64
    n3, B3 = c3.numel, c3.block
    x3 = to_dev(c3.weight())
    q3c = torch.empty(n3, dtype=torch.uint8, device=dev)
    q3s = torch.empty(n3 // B3, dtype=torch.float32, device=dev)
    z.zpp_quantize_blocks(x3, z.ZPP_BF16, n3, B3, 8, q3c, q3s)
    del x3
    y3 = torch.empty(n3, dtype=torch.bfloat16, device=dev)
    res[c3.name] = rows([
        ("dequantize_int8_b2048_64_shards", (q3c, q3s, y3),
         lambda b: z.zpp_dequantize_blocks(b[0], b[1], 8, n3, B3, b[2], z.ZPP_BF16), n3 + 4 * n3 // B3, 2 * n3),
    ])
    del y3
    # the same codes to binary32 (a full-precision copy of the weights)
    y3f = torch.empty(n3, dtype=torch.float32, device=dev)
    res[c3.name].update(rows([
        ("dequantize_int8_b2048_64_shards_f32", (q3c, q3s, y3f),
         lambda b: z.zpp_dequantize_blocks(b[0], b[1], 8, n3, B3, b[2], z.ZPP_FP32), n3 + 4 * n3 // B3, 4 * n3),
    ]))
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def block_sweep(torch, z, K: int = 10) -> dict:
    """Kernel time and quantization error for every block size on the GQA weight.

    The error of block quantization is compared with one scale for the whole
    tensor (global quantization; page "Quantized LLM Training at Scale with
    ZeRO++", pillar 1 QWZ, credits block quantization with 3.3x better
    precision than global). Error = root mean square of dequantize(quantize(x)) - x,
    with the dequantized values from the library in binary32; the global
    reference is the same rule applied with torch, for comparison only.
    """
    import synth

    w = synth.gqa_weight()
    x = torch.from_numpy(w).view(torch.int16).view(torch.bfloat16).cuda()
    n = x.numel()
    stream = torch.cuda.current_stream()
    chunk = 1 << 26

    def rms_err(y):
        acc = 0.0
        for i in range(0, n, chunk):
            d = y[i:i + chunk].double() - x[i:i + chunk].double()
            acc += float((d * d).sum())
        return (acc / n) ** 0.5

    a = x.float().abs().max()
    rows, global_rms = [], {}
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    yb = torch.empty_like(x)
    for bits in (8, 4):
        Q = 127.0 if bits == 8 else 7.0
        sg = (a / Q).float()
        for i in range(0, n, chunk):
            xi = x[i:i + chunk].float()
            y[i:i + chunk] = torch.round(xi / sg).clamp_(-Q, Q) * sg
        global_rms[str(bits)] = rms_err(y)
        codes = torch.empty(n * bits // 8, dtype=torch.uint8, device="cuda")
        for lb in range(5, 13):
            B = 1 << lb
            scales = torch.empty(n // B, dtype=torch.float32, device="cuda")
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * K)]
            z.zpp_quantize_blocks(x, z.ZPP_BF16, n, B, bits, codes, scales)
            z.zpp_dequantize_blocks(codes, scales, bits, n, B, yb, z.ZPP_BF16)
            for k in range(K):
                ev[2 * k][0].record(stream)
                z.zpp_quantize_blocks(x, z.ZPP_BF16, n, B, bits, codes, scales)
                ev[2 * k][1].record(stream)
                ev[2 * k + 1][0].record(stream)
                z.zpp_dequantize_blocks(codes, scales, bits, n, B, yb, z.ZPP_BF16)
                ev[2 * k + 1][1].record(stream)
            torch.cuda.synchronize()
            qms = sum(ev[2 * k][0].elapsed_time(ev[2 * k][1]) for k in range(K)) / K
            dms = sum(ev[2 * k + 1][0].elapsed_time(ev[2 * k + 1][1]) for k in range(K)) / K
            cb, sb = n * bits // 8, 4 * (n // B)
            z.zpp_dequantize_blocks(codes, scales, bits, n, B, y, z.ZPP_FP32)
            torch.cuda.synchronize()
            err = rms_err(y)
            rows.append({
                "bits": bits, "block": B,
                "quantize_ms": round(qms, 4),
                "quantize_hbm_frac": round((2 * n + cb + sb) / (qms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "dequantize_ms": round(dms, 4),
                "dequantize_hbm_frac": round((cb + sb + 2 * n) / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "rms_error": err,
                "global_over_block_rms": round(global_rms[str(bits)] / err, 3),
            })
            log(f"bits {bits} B {B}: quantize {qms:.3f} ms, dequantize {dms:.3f} ms, rms {err:.3e}")
            del scales
        del codes
    return {"tensor": f"GQA layer weight, {n:,} bf16, N(0, 0.01) with 0.01% outliers x100",
            "global_rms_error": global_rms, "rows": rows}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--block-sweep", action="store_true",
                    help="instead of the step: time and error of every block size on the GQA weight")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the step: kernel times at the three smaller workload shapes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the codec and runs on exactly one GPU; "
              f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported: collectives are out of scope "
              "and every rank's work is the same per-GPU kernel sequence.", file=sys.stderr)
        return 2

    import torch

    import block_quantization_codec_amd as z

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)

    if args.block_sweep:
        print(json.dumps({"block_sweep": block_sweep(torch, z)}), flush=True)
        return 0
    if args.configs:
        print(json.dumps({"configs": configs_bench(torch, z)}), flush=True)
        return 0

    # plain copy of known size, for scaling the rocprofv3 byte counters
    cal_src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    step = Step(torch, z)
    fns = step.launches()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()

    K = args.steps
    # the step as a caller runs it: K steps back to back, nothing in between
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        for f in fns:
            f()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K

    # the same step captured once into a HIP graph and replayed K times (a
    # caller that replays a fixed sequence pays no per-launch host work)
    graph_ms = graph_step_ms(torch, fns, K)

    # the same K steps again with HIP events around every kernel row
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        for i, f in enumerate(fns):
            ev[k][i][0].record(stream)
            f()
            ev[k][i][1].record(stream)
    torch.cuda.synchronize()

    per, spread = [], {}
    for i, (name, fam, rin, wout, kname) in enumerate(step.kernels):
        times = sorted(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(K))
        ms = sum(times) / K
        per.append((name, fam, rin, wout, kname, ms))
        spread[name] = {"ms_p10": round(times[int(0.1 * (K - 1))], 5), "ms_p50": round(times[(K - 1) // 2], 5),
                        "ms_p90": round(times[int(0.9 * (K - 1) + 0.5)], 5)}
    total_in = sum(p[2] for p in per)
    total_rw = sum(p[2] + p[3] for p in per)
    value = total_in / (ms_per_step * 1e-3) / 1e9

    dom = max(per, key=lambda p: p[5])
    name, fam, rin, wout, kname, ms = dom
    achieved = (rin + wout) / (ms * 1e-3) / 1e9
    traffic = traffic_record(name, fam)
    roofline = {
        "bound": "hbm",
        "kernel": name,
        "rocprof_name": kname,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "algorithmic_bytes": rin + wout,
        "avg_launch_ms": round(ms, 5),
    }

    # timed after the steps, not part of them: the unfused reorder + quantize
    # pair, and hop 2 writing the averaged (optimizer-ready) shard
    unfused = time_rows(torch, stream, step.unfused_launches(), step.unfused_kernels, K)
    extra = time_rows(torch, stream, step.extra_launches(), step.extra_kernels, K)
    copy = copy_ceiling(torch, z, stream, K)
    # rows that move less than 1 GiB: also against a plain copy of their own size
    same = {p[0]: same_size_copy(torch, z, stream, p[2] + p[3], K) for p in per if p[2] + p[3] < (1 << 30)}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(step)

    line = {
        "metric": "quantize / dequant-reduce-requant input GB/s and % of HBM peak, 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("qgZ 32x8 rank-255 share of a 500M-element bf16 gradient bucket (slice reorder fused "
                         "into the int4 B=256 quantize, 8-way hop-1 dequant-reduce-requant, 32-way hop-2 fp32 "
                         "reduce) + "
                         "qwZ/qgZ on one 855,638,016-parameter GQA layer (int8 B=512 quantize and "
                         "dequantize of the weight, int4 B=128 quantize of the gradient)"),
            "bucket_elems": c_bucket(step),
            "gqa_layer_elems": step.W.numel(),
            "topology": "32 nodes x 8 GPUs (simulated; one GPU's share)",
            "parallelism": "none (one GPU's share of ZeRO++ data parallelism)",
        },
        "hbm_frac_step": round(total_rw / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels": {p[0]: {"ms": round(p[5], 5), **spread[p[0]], "in_GBps": round(p[2] / (p[5] * 1e-3) / 1e9, 1),
                           "rw_GBps": round((p[2] + p[3]) / (p[5] * 1e-3) / 1e9, 1),
                           "hbm_frac": round((p[2] + p[3]) / (p[5] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                           "copy_frac": round((p[2] + p[3]) / (p[5] * 1e-3) / 1e9 / copy["GBps"], 4),
                           **({"copy_same_size_ms": round(same[p[0]], 5),
                               "of_copy_same_size": round(same[p[0]] / p[5], 4)} if p[0] in same else {})}
                    for p in per},
        "copy_ceiling": copy,
        "graph_step": {"ms_per_step": round(graph_ms, 4),
                       "value": round(total_in / (graph_ms * 1e-3) / 1e9, 2),
                       "what": "the same step captured once into a HIP graph, replayed K times"},
        "unfused_reorder_then_quantize": unfused,
        "beside_the_step": extra,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def c_bucket(step) -> int:
    return step.c.numel


if __name__ == "__main__":
    sys.exit(main())
