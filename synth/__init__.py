"""Seeded synthetic inputs for the ZeRO++ block-quantization codec workloads.

This module only *draws* inputs: shapes, value distributions, outlier
positions, the zero padding of a gradient bucket, and the workload
definitions. It holds none of the codec's arithmetic (no block maxima, no
scales, no codes, no reorder, no reductions), so both the CPU oracle and the
GPU library can be fed from it without sharing code with each other.

Every array comes from ``numpy.random.default_rng`` keyed by
``[seed, workload_id, tensor_id, rank, chunk]``. Large tensors are drawn in
fixed-size chunks, each chunk from its own key, so the result does not depend
on how many threads draw them. Values are drawn in float32 (or float64 for
Student-t, then cast), scaled, given their outliers, and rounded to bfloat16
with torch's round-to-nearest-even cast. bfloat16 tensors are returned as
``numpy.uint16`` bit patterns.

Workloads (sizes as the ZeRO++ codec is exercised on one GPU; no dataset is
involved anywhere, every value is synthetic):

* ``qwz_int8_4096x4096`` - one bf16 weight 4096x4096, N(0, 0.02) with 0.1 %
  of positions multiplied by 50, int8, block 256.
* ``qgz_int4_2x4_16M`` - 8 simulated ranks (2 nodes x 4 GPUs), 16,000,000
  bf16 gradient elements each, N(0, 1e-3), int4, block 128.
* ``qwz_dequant_64x_llama_layer`` - one Llama-style layer (hidden 4096, FFN
  11008; q,k,v,o,gate,up,down = 202,375,168 weights) split into 64 shards,
  values as the 4096x4096 weight, int8, block 2048.
* ``qgz_int4_32x8_500M`` - one GPU's 500,000,000-element bf16 gradient
  bucket, Student-t(nu=3) x 1e-4, 32 nodes x 8 GPUs, int4, block 256; the
  bucket is zero-padded to 256 equal block-aligned slices.
* ``gqa_layer_8192_int8w_int4g`` - one GQA layer (hidden 8192, 64 query /
  8 key-value heads of 128, FFN 28672; 855,638,016 weights) as a bf16 weight
  and an independent bf16 gradient, N(0, 0.01) with 0.01 % of positions
  multiplied by 100; weight int8 block 512, gradient int4 block 128.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 0
CHUNK = 1 << 22  # elements per independently keyed draw


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) via torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _chunked(n: int, key: tuple, fill) -> np.ndarray:
    """Draw ``n`` float32 values chunk by chunk; ``fill(rng, count)`` draws one chunk."""
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, CHUNK))

    def work(ci: int) -> None:
        s = starts[ci]
        e = min(n, s + CHUNK)
        rng = np.random.default_rng([*key, ci])
        out[s:e] = fill(rng, e - s)

    if len(starts) <= 1:
        for ci in range(len(starts)):
            work(ci)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))
    return out


def normal_f32(n: int, sigma: float, key: tuple) -> np.ndarray:
    sig = np.float32(sigma)
    return _chunked(n, key, lambda rng, c: rng.standard_normal(c, dtype=np.float32) * sig)


def student_t_f32(n: int, nu: float, scale: float, key: tuple) -> np.ndarray:
    sc = np.float32(scale)
    return _chunked(n, key, lambda rng, c: rng.standard_t(nu, c).astype(np.float32) * sc)


def sum_of_student_t_f32(n: int, nu: float, scale: float, terms: int, key: tuple) -> np.ndarray:
    """Each value is the sum of ``terms`` independent Student-t draws times ``scale``.

    Stands in for a partial gradient sum that another node reduced over its
    GPUs before sending it on (drawn in float64, then cast to float32).
    """

    def fill(rng, c):
        acc = np.zeros(c, dtype=np.float64)
        for _ in range(terms):
            acc += rng.standard_t(nu, c)
        return (acc * scale).astype(np.float32)

    return _chunked(n, key, fill)


def add_outliers(x: np.ndarray, frac: float, mult: float, key: tuple) -> np.ndarray:
    """Multiply round(frac * n) distinct, uniformly chosen positions by ``mult`` (sign kept)."""
    k = int(round(frac * x.size))
    if k:
        rng = np.random.default_rng([*key, 0x0ff1])
        pos = rng.choice(x.size, k, replace=False)
        x[pos] *= np.float32(mult)
    return x


def bf16_normal(n: int, sigma: float, key: tuple, outlier_frac: float = 0.0,
                outlier_mult: float = 1.0) -> np.ndarray:
    x = normal_f32(n, sigma, key)
    add_outliers(x, outlier_frac, outlier_mult, key)
    return _f32_to_bf16_bits(x)


def bf16_student_t(n: int, nu: float, scale: float, key: tuple, pad_to: int | None = None) -> np.ndarray:
    """Student-t bf16 values; if ``pad_to`` is given the result is zero-padded to that length."""
    x = student_t_f32(n, nu, scale, key)
    b = _f32_to_bf16_bits(x)
    if pad_to is not None and pad_to > n:
        b = np.concatenate([b, np.zeros(pad_to - n, dtype=np.uint16)])
    return b


# --------------------------------------------------------------------------
# workload definitions
# --------------------------------------------------------------------------


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def padded_slice_len(numel: int, n_slices: int, block: int) -> int:
    """Length of each of ``n_slices`` equal slices holding ``numel`` elements,
    each slice a whole number of blocks (only the last slice carries padding)."""
    return ceil_div(ceil_div(numel, n_slices), block) * block


@dataclass(frozen=True)
class QwzWeight:
    """A bf16 weight quantized for the forward all-gather."""

    name: str
    wid: int
    numel: int
    block: int
    bits: int
    sigma: float
    outlier_frac: float
    outlier_mult: float
    shards: int = 1

    def weight(self, tensor_id: int = 0) -> np.ndarray:
        return bf16_normal(self.numel, self.sigma, (SEED, self.wid, tensor_id, 0),
                           self.outlier_frac, self.outlier_mult)


@dataclass(frozen=True)
class QgzBucket:
    """A gradient bucket on the qgZ two-hop path (n_nodes x gpus_per_node ranks)."""

    name: str
    wid: int
    numel: int          # real elements per rank
    block: int
    bits: int
    n_nodes: int
    gpus_per_node: int
    dist: str           # "normal" or "student_t"
    sigma: float = 0.0  # normal
    nu: float = 0.0     # student_t
    scale: float = 0.0  # student_t
    ranks_simulated: tuple = field(default_factory=tuple)

    @property
    def n_ranks(self) -> int:
        return self.n_nodes * self.gpus_per_node

    @property
    def slice_len(self) -> int:
        return padded_slice_len(self.numel, self.n_ranks, self.block)

    @property
    def padded(self) -> int:
        return self.slice_len * self.n_ranks

    @property
    def chunk_len(self) -> int:
        """Elements a rank sends to each local peer in the intra-node hop."""
        return self.slice_len * self.n_nodes

    def bucket(self, rank: int, tensor_id: int = 0) -> np.ndarray:
        """Rank ``rank``'s own bf16 gradient bucket, zero-padded to ``padded``."""
        key = (SEED, self.wid, tensor_id, rank)
        if self.dist == "normal":
            b = bf16_normal(self.numel, self.sigma, key)
            if self.padded > self.numel:
                b = np.concatenate([b, np.zeros(self.padded - self.numel, np.uint16)])
            return b
        return bf16_student_t(self.numel, self.nu, self.scale, key, pad_to=self.padded)

    def real_in_slice(self, slice_index: int) -> int:
        """How many of a slice's elements are real data (the rest is padding)."""
        s0 = slice_index * self.slice_len
        return max(0, min(self.slice_len, self.numel - s0))

    def peer_chunk(self, local_peer: int, dest_local: int, node: int) -> np.ndarray:
        """bf16 chunk that local peer ``local_peer`` sends to ``dest_local`` in hop 1.

        It is a fresh draw of the bucket's distribution, laid out like chunk
        ``dest_local`` of a reordered bucket: its tail (the padded slice, when
        the chunk holds one) is zero.
        """
        key = (SEED, self.wid, 100 + local_peer, node * self.gpus_per_node + dest_local)
        n = self.chunk_len
        if self.dist == "normal":
            v = _f32_to_bf16_bits(normal_f32(n, self.sigma, key))
        else:
            v = _f32_to_bf16_bits(student_t_f32(n, self.nu, self.scale, key))
        # Positions of this chunk that hold padding after the reorder: the chunk
        # for local rank j holds slices k*g + j (k = 0..n_nodes-1) in order.
        for k in range(self.n_nodes):
            real = self.real_in_slice(k * self.gpus_per_node + dest_local)
            if real < self.slice_len:
                v[k * self.slice_len + real:(k + 1) * self.slice_len] = 0
        return v

    def node_partial(self, src_node: int, dest_node: int, dest_local: int) -> np.ndarray:
        """float32 partial sum that node ``src_node`` sends to rank (dest_node, dest_local)
        in hop 2: one slice, a sum of gpus_per_node independent draws (zero where
        the slice is padding)."""
        key = (SEED, self.wid, 1000 + src_node, dest_node * self.gpus_per_node + dest_local)
        n = self.slice_len
        if self.dist == "normal":
            v = _chunked(n, key, lambda rng, c: (rng.standard_normal((self.gpus_per_node, c))
                                                 .sum(axis=0) * self.sigma).astype(np.float32))
        else:
            v = sum_of_student_t_f32(n, self.nu, self.scale, self.gpus_per_node, key)
        real = self.real_in_slice(dest_node * self.gpus_per_node + dest_local)
        v[real:] = 0
        return v


QWZ_INT8_4096 = QwzWeight("qwz_int8_4096x4096", 1, 4096 * 4096, 256, 8, 0.02, 1e-3, 50.0)

QGZ_INT4_2x4 = QgzBucket("qgz_int4_2x4_16M", 2, 16_000_000, 128, 4, 2, 4, "normal", sigma=1e-3)

LLAMA_LAYER = 4 * 4096 * 4096 + 3 * 4096 * 11008  # q,k,v,o + gate,up,down
QWZ_DEQUANT_64 = QwzWeight("qwz_dequant_64x_llama_layer", 3, LLAMA_LAYER, 2048, 8, 0.02, 1e-3, 50.0,
                           shards=64)

QGZ_INT4_32x8 = QgzBucket("qgz_int4_32x8_500M", 4, 500_000_000, 256, 4, 32, 8, "student_t",
                          nu=3.0, scale=1e-4)

GQA_LAYER = 2 * 8192 * 8192 + 2 * 8192 * 1024 + 3 * 8192 * 28672  # q,o + k,v + gate,up,down
GQA_W_INT8 = QwzWeight("gqa_layer_8192_weight_int8", 5, GQA_LAYER, 512, 8, 0.01, 1e-4, 100.0)
GQA_G_INT4 = QwzWeight("gqa_layer_8192_grad_int4", 5, GQA_LAYER, 128, 4, 0.01, 1e-4, 100.0)

WORKLOADS = {w.name: w for w in (QWZ_INT8_4096, QGZ_INT4_2x4, QWZ_DEQUANT_64, QGZ_INT4_32x8,
                                 GQA_W_INT8, GQA_G_INT4)}


def gqa_weight() -> np.ndarray:
    return GQA_W_INT8.weight(tensor_id=0)


def gqa_grad() -> np.ndarray:
    # independent of the weight: its own tensor id
    return GQA_G_INT4.weight(tensor_id=1)


def small_bf16(n: int, key: tuple, sigma: float = 1.0, outlier_frac: float = 0.0,
               outlier_mult: float = 1.0) -> np.ndarray:
    """Small bf16 test tensor (single keyed draw)."""
    rng = np.random.default_rng(list(key))
    x = (rng.standard_normal(n, dtype=np.float32) * np.float32(sigma))
    add_outliers(x, outlier_frac, outlier_mult, key)
    return _f32_to_bf16_bits(x)


def small_f32(n: int, key: tuple, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(list(key))
    return rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)


def random_codes(nbytes: int, key: tuple) -> np.ndarray:
    """Uniform random code bytes (any bit pattern)."""
    rng = np.random.default_rng(list(key))
    return rng.integers(0, 256, nbytes, dtype=np.uint8)


def random_scales(n: int, key: tuple, lo: float = 1e-6, hi: float = 1e-2) -> np.ndarray:
    rng = np.random.default_rng(list(key))
    return np.exp(rng.uniform(np.log(lo), np.log(hi), n)).astype(np.float32)
