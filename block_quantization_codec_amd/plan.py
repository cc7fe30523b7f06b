"""Host-side sizing for the codec: buffer layout of the qgZ exchange, and the
ZeRO / ZeRO++ memory and communication volume formulas the pages state.

Pure arithmetic on sizes; it launches nothing and needs no GPU.

Sources (pages as published, by title and section):
  [Z++ vol]  "Quantized LLM Training at Scale with ZeRO++", section
             "Understanding the ZeRO-3 Communication Volume": ZeRO-3 moves
             three times the model size per iteration (forward all-gather M,
             backward all-gather M, gradient reduce-scatter M); ZeRO++ cuts
             that to 0.75 M.
  [Z++ 3P]   same page, "The Three Pillars of ZeRO++": qwZ sends 8-bit
             weights (M -> 0.5 M), hpZ keeps a secondary weight partition in
             the node so the backward all-gather crosses no node (M -> 0),
             qgZ sends 4-bit gradients through a two-hop all-to-all
             (M -> 0.25 M) after a tensor-slice reorder.
  [Z123]     "ZeRO-1/2/3", section on the three stages: per-GPU memory
             4 Phi + 12 Phi / N_d (stage 1), 2 Phi + 14 Phi / N_d (stage 2),
             16 Phi / N_d (stage 3) for mixed precision with Adam (16 bytes
             per parameter unsharded); stage 3 communicates 3 Phi per GPU
             against 2 Phi for plain data parallelism.
  [ZS2]      "ZeRO Stage 2: Gradient Partitioning", the stage-2 memory
             equation M = 2 Psi + (2 Psi + 12 Psi) / N_d.

Units: Phi (or Psi) is the parameter count; memory is in bytes. Volumes are
in units of M, the model size in 16-bit bytes (2 Phi bytes), as the ZeRO++
page counts them.
"""
from __future__ import annotations

from dataclasses import dataclass

BYTES_PER_PARAM_UNSHARDED = 16  # fp16 weights 2 + fp16 gradients 2 + fp32 Adam state 12 [Z123]
OPTIMIZER_BYTES_PER_PARAM = 12  # fp32 master weights, momentum and variance [Z123]


# ---- ZeRO memory per GPU --------------------------------------------------

def zero_memory_per_gpu(params: int, n_d: int, stage: int) -> float:
    """Bytes per GPU for mixed-precision Adam at ZeRO `stage` (0 = plain data
    parallelism) over `n_d` data-parallel GPUs [Z123] [ZS2]."""
    if n_d < 1 or params < 0:
        raise ValueError("need params >= 0 and n_d >= 1")
    P, K = float(params), float(OPTIMIZER_BYTES_PER_PARAM)
    if stage == 0:
        return (2 + 2 + K) * P
    if stage == 1:
        return 2 * P + 2 * P + K * P / n_d
    if stage == 2:
        return 2 * P + (2 * P + K * P) / n_d
    if stage == 3:
        return (2 * P + 2 * P + K * P) / n_d
    raise ValueError("stage must be 0, 1, 2 or 3")


# ---- communication volume per GPU and iteration ------------------------------

def zero_comm_volume(stage: int) -> float:
    """Per-GPU communication per iteration, in units of M, for plain data
    parallelism and ZeRO stages 1-3 [Z123]: an all-reduce is a reduce-scatter
    plus an all-gather (2 M); stage 3 adds a second weight all-gather (3 M)."""
    if stage in (0, 1, 2):
        return 2.0
    if stage == 3:
        return 3.0
    raise ValueError("stage must be 0, 1, 2 or 3")


@dataclass(frozen=True)
class ZeroPPVolume:
    """ZeRO++ per-GPU volume per iteration, in units of M [Z++ vol] [Z++ 3P]."""
    forward_weights: float   # qwZ all-gather of quantized weights
    backward_weights: float  # hpZ: all-gather inside the node only (0 across nodes)
    gradients: float         # qgZ two-hop all-to-all of quantized gradients
    zero3_total: float = 3.0

    @property
    def total(self) -> float:
        return self.forward_weights + self.backward_weights + self.gradients

    @property
    def reduction(self) -> float:
        return self.zero3_total / self.total


def quantized_fraction(bits: int, block: int | None) -> float:
    """Bytes of `bits`-bit codes plus one binary32 scale per `block` elements,
    as a fraction of 16-bit bytes; block None ignores the scales."""
    if bits not in (8, 4):
        raise ValueError("bits must be 8 or 4")
    codes = bits / 16.0
    return codes if block is None else codes + 4.0 / (2.0 * block)


def zeropp_volume(weight_bits: int = 8, grad_bits: int = 4, weight_block: int | None = None,
                  grad_block: int | None = None, hpz: bool = True) -> ZeroPPVolume:
    """ZeRO++'s three communication steps in units of M. Without block sizes
    this is the pages' count (0.5 M + 0 + 0.25 M = 0.75 M); with them the
    per-block scales are included."""
    return ZeroPPVolume(forward_weights=quantized_fraction(weight_bits, weight_block),
                        backward_weights=0.0 if hpz else 1.0,
                        gradients=quantized_fraction(grad_bits, grad_block))


# ---- qgZ exchange layout ---------------------------------------------------

@dataclass(frozen=True)
class QgzLayout:
    """Sizes (elements and bytes) of the buffers of one qgZ reduce-scatter.

    The bucket of `numel` elements is zero-padded to N = n_nodes * gpus_per_node
    equal slices of `slice_elems` (a whole number of blocks, as small as that
    allows). Hop 1 receives gpus_per_node chunks of n_nodes slices; hop 2
    receives n_nodes slices; the owner keeps one slice. Ranks are node-major.
    """
    numel: int
    n_nodes: int
    gpus_per_node: int
    block: int
    bits: int
    slice_elems: int

    @property
    def n_ranks(self) -> int:
        return self.n_nodes * self.gpus_per_node

    @property
    def padded_elems(self) -> int:
        return self.slice_elems * self.n_ranks

    @property
    def chunk_elems(self) -> int:
        """Elements each local rank receives from every local peer in hop 1."""
        return self.slice_elems * self.n_nodes

    def code_bytes(self, elems: int) -> int:
        return elems * self.bits // 8

    def scale_count(self, elems: int) -> int:
        return elems // self.block

    def wire_bytes(self, elems: int) -> int:
        """Codes plus binary32 scales of `elems` elements."""
        return self.code_bytes(elems) + 4 * self.scale_count(elems)

    @property
    def hop1_recv_bytes(self) -> int:
        return self.gpus_per_node * self.wire_bytes(self.chunk_elems)

    @property
    def hop2_recv_bytes(self) -> int:
        return self.n_nodes * self.wire_bytes(self.slice_elems)

    @property
    def intra_node_send_bytes(self) -> int:
        """Hop-1 bytes one GPU sends to its g - 1 local peers."""
        return (self.gpus_per_node - 1) * self.wire_bytes(self.chunk_elems)

    @property
    def inter_node_send_bytes(self) -> int:
        """Hop-2 bytes one GPU sends to its n - 1 peers on other nodes."""
        return (self.n_nodes - 1) * self.wire_bytes(self.slice_elems)

    def slice_of_rank(self, rank: int) -> tuple[int, int]:
        """[start, end) of the padded bucket that `rank` owns after hop 2."""
        return rank * self.slice_elems, (rank + 1) * self.slice_elems

    def real_elems_of_rank(self, rank: int) -> int:
        """Elements of `rank`'s slice that are not padding."""
        s0, s1 = self.slice_of_rank(rank)
        return max(0, min(s1, self.numel) - s0)


def qgz_layout(numel: int, n_nodes: int, gpus_per_node: int, block: int, bits: int = 4) -> QgzLayout:
    """Layout of one bucket: slice = the smallest multiple of `block` with
    N * slice >= numel (zero padding at the tail keeps every scale and sum)."""
    if numel < 0 or n_nodes < 1 or gpus_per_node < 1:
        raise ValueError("need numel >= 0, n_nodes >= 1, gpus_per_node >= 1")
    if block < 1 or block & (block - 1):
        raise ValueError("block must be a power of two")
    if bits not in (8, 4):
        raise ValueError("bits must be 8 or 4")
    n = n_nodes * gpus_per_node
    per = -(-numel // n)
    slice_elems = -(-per // block) * block
    return QgzLayout(numel, n_nodes, gpus_per_node, block, bits, slice_elems)
