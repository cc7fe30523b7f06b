"""GPU parity of zpp_dequant_reduce_requant_split against the CPU oracle.

The split hop-1 step writes the requantized codes and scales of a kept
window of blocks to one buffer and everything else, in order and with the
window left out, to another (page "Quantized LLM Training at Scale with
ZeRO++", section "The Three Pillars of ZeRO++", QGZ: after the intra-node
reduction each GPU sends all but its own sub-chunk across nodes). The
expected bytes are the oracle's unsplit hop result, cut the same way on the
host. Covers windows at the start, middle and end, empty and whole windows,
both lane layouts (8 and 32 elements per lane, the latter with 4-bit code
vectors landing in LDS), 4- and 8-bit codes, input counts that end in a
partial batch, and a window that straddles the 2^29-element boundary
between two launches. Every output sits between canary bytes.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle_par
import synth
from gpu_util import Guarded, assert_bits_equal, dev, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _inputs(R, bits_in, numel, block, seed, random_bytes=False):
    """R inputs side by side: quantized by the oracle from Student-t data, or
    arbitrary code bytes with scales spread over fifteen binades."""
    per_c, per_s = numel * bits_in // 8, numel // block
    if random_bytes:
        rng = np.random.default_rng([seed, R, numel, block, bits_in])
        codes = rng.integers(0, 256, R * per_c, dtype=np.uint8)
        scales = np.exp2(rng.uniform(-20, -5, R * per_s)).astype(np.float32)
        return codes, per_c, scales, per_s
    codes = np.empty(R * per_c, np.uint8)
    scales = np.empty(R * per_s, np.float32)
    for r in range(R):
        x = synth.bf16_student_t(numel, 3.0, 1e-4 * (1 + r % 3), (seed, r, numel, block))
        c, s = oracle_par.quantize(x, block, bits_in)
        codes[r * per_c:(r + 1) * per_c] = c
        scales[r * per_s:(r + 1) * per_s] = s
    return codes, per_c, scales, per_s


def _split(R, bits_in, bits_out, numel, block, keep_begin, keep_elems, seed=5, random_bytes=False):
    import block_quantization_codec_amd as z
    codes, pc, scales, ps = _inputs(R, bits_in, numel, block, seed, random_bytes)
    send = numel - keep_elems
    gsc = Guarded(send * bits_out // 8) if send else None
    gss = Guarded(4 * (send // block)) if send else None
    gkc = Guarded(keep_elems * bits_out // 8) if keep_elems else None
    gks = Guarded(4 * (keep_elems // block)) if keep_elems else None
    ci, si = dev(codes), dev(scales)
    torch.cuda.synchronize()
    z.zpp_dequant_reduce_requant_split(ci, pc, si, ps, R, bits_in, numel, block, keep_begin, keep_elems,
                                       gsc.ptr if gsc else None, gss.ptr if gss else None,
                                       gkc.ptr if gkc else None, gks.ptr if gks else None, bits_out)
    torch.cuda.synchronize()
    for g in (gsc, gss, gkc, gks):
        if g is not None:
            assert g.untouched(), "write outside an output buffer"
    cl = [codes[r * pc:(r + 1) * pc] for r in range(R)]
    sl = [scales[r * ps:(r + 1) * ps] for r in range(R)]
    co, so, _ = oracle_par.dequant_reduce_requant(cl, sl, bits_in, numel, block, bits_out)
    k0, k1 = keep_begin, keep_begin + keep_elems

    def cut_codes(a, lo, hi):
        return a[lo * bits_out // 8:hi * bits_out // 8]

    def cut_scales(a, lo, hi):
        return a[lo // block:hi // block]

    what = f"R={R} in={bits_in} out={bits_out} B={block} n={numel} keep=[{k0},{k1})"
    if keep_elems:
        assert_bits_equal(gks.as_np(np.float32), cut_scales(so, k0, k1), "keep scales " + what)
        assert_bits_equal(gkc.bytes(), cut_codes(co, k0, k1), "keep codes " + what)
    if send:
        want_c = np.concatenate([cut_codes(co, 0, k0), cut_codes(co, k1, numel)])
        want_s = np.concatenate([cut_scales(so, 0, k0), cut_scales(so, k1, numel)])
        assert_bits_equal(gss.as_np(np.float32), want_s, "send scales " + what)
        assert_bits_equal(gsc.bytes(), want_c, "send codes " + what)


# the 8-element layout (small outputs) and the 32-element layout (4096+ tiles
# of 2048 elements)
SMALL = 96 * 256
WIDE = 4096 * 2048 + 7 * 256


@pytest.mark.parametrize("numel", [SMALL, WIDE])
@pytest.mark.parametrize("where", ["start", "middle", "end", "none", "all", "tile_ends", "within_one_tile"])
def test_window_positions(numel, where):
    """Tiles are 512 elements in the 8-element layout (SMALL) and 2048 in the
    32-element one (WIDE). A tile lies before, after or inside the window,
    or holds one or both of its ends; "tile_ends" puts both ends on tile
    boundaries (no tile holds an end), "within_one_tile" both ends inside
    the same tile (with 2-block tiles: one block, from mid-tile to the
    tile's end)."""
    B = 256
    tile = 512 if numel == SMALL else 2048
    w = {"start": (0, 31 * B), "middle": (numel // 2 // B * B, 5 * B), "end": (numel - 9 * B, 9 * B),
         "none": (numel // B // 3 * B, 0), "all": (0, numel),
         "tile_ends": (numel // 2 // tile * tile, 4 * tile),
         "within_one_tile": (numel // 3 // tile * tile + B, max(tile - 2 * B, B))}[where]
    _split(8, 4, 4, numel, B, *w)


@pytest.mark.parametrize("bits_in,bits_out,R,block", [(4, 4, 9, 128), (8, 8, 3, 256), (4, 8, 17, 512),
                                                       (8, 4, 5, 32), (4, 4, 1, 2048), (4, 4, 8, 4096),
                                                       (4, 4, 16, 32)])
@pytest.mark.parametrize("numel_kind", ["small", "wide"])
def test_widths_blocks_and_input_counts(bits_in, bits_out, R, block, numel_kind):
    numel = (96 * block if numel_kind == "small" else 4096 * 2048 + 3 * max(block, 2048))
    keep_begin = (numel // block // 4) * block
    _split(R, bits_in, bits_out, numel, block, keep_begin, 3 * block, random_bytes=True)


def test_hop1_shape_of_the_32x8_share():
    """Hop 1 as the 32x8 share launches it: 8 inputs of a 62.5M-element chunk
    cut into 32 sub-chunks of 1,953,280; the rank on the last node keeps the
    last sub-chunk."""
    c = synth.QGZ_INT4_32x8
    S, C = c.slice_len, c.chunk_len
    _split(8, 4, 4, C, c.block, C - S, S, seed=11)


def test_window_across_the_launch_boundary():
    """Outputs past 2^29 elements take two launches; the kept window straddles
    the boundary between them."""
    numel = (1 << 29) + (1 << 20)
    B = 256
    _split(2, 4, 4, numel, B, (1 << 29) - 64 * B, 128 * B, seed=12, random_bytes=True)


def test_empty_is_a_no_op():
    import block_quantization_codec_amd as z
    z.zpp_dequant_reduce_requant_split(None, 0, None, 0, 4, 4, 0, 256, 0, 0, None, None, None, None, 4)


def test_split_matches_the_unsplit_call_on_random_code_bytes():
    """Arbitrary code bytes and scales over several binades: both halves equal
    the unsplit call's output (library against library, beside the oracle
    comparisons above)."""
    import block_quantization_codec_amd as z
    R, B = 9, 128
    numel = 4096 * 2048 + 11 * B
    rng = np.random.default_rng([77, R])
    codes = dev(rng.integers(0, 256, R * numel // 2, dtype=np.uint8))
    scales = dev(np.exp2(rng.uniform(-30, 10, R * (numel // B))).astype(np.float32))
    full_c, full_s, _ = z.dequant_reduce_requant(codes, scales, R, 4, numel, B, bits_out=4, want_sum=False)
    k0, kl = 1000 * B, 77 * B
    sc = torch.empty((numel - kl) // 2, dtype=torch.uint8, device="cuda")
    ss = torch.empty((numel - kl) // B, dtype=torch.float32, device="cuda")
    kc = torch.empty(kl // 2, dtype=torch.uint8, device="cuda")
    ks = torch.empty(kl // B, dtype=torch.float32, device="cuda")
    z.zpp_dequant_reduce_requant_split(codes, numel // 2, scales, numel // B, R, 4, numel, B, k0, kl, sc, ss, kc, ks, 4)
    torch.cuda.synchronize()
    fc, fs = full_c.cpu().numpy(), full_s.cpu().numpy()
    assert_bits_equal(kc.cpu().numpy(), fc[k0 // 2:(k0 + kl) // 2], "keep codes")
    assert_bits_equal(ks.cpu().numpy(), fs[k0 // B:(k0 + kl) // B], "keep scales")
    assert_bits_equal(sc.cpu().numpy(), np.concatenate([fc[:k0 // 2], fc[(k0 + kl) // 2:]]), "send codes")
    assert_bits_equal(ss.cpu().numpy(), np.concatenate([fs[:k0 // B], fs[(k0 + kl) // B:]]), "send scales")
    # and the unsplit hop sum against the oracle on these bytes
    cl = codes.cpu().numpy().reshape(R, -1)
    sl = scales.cpu().numpy().reshape(R, -1)
    co, so, _ = oracle.dequant_reduce_requant(list(cl), list(sl), 4, numel, B, 4)
    assert_bits_equal(fc, co, "unsplit codes vs oracle")
    assert_bits_equal(fs, so, "unsplit scales vs oracle")


def test_tensor_helper_matches_the_raw_entry_point():
    """block_quantization_codec_amd.dequant_reduce_requant_split (outputs
    allocated by the binding) equals the oracle's requantized sum, cut at the
    window, for a hop of 8 inputs and for a window covering everything."""
    import block_quantization_codec_amd as z
    R, B = 8, 256
    numel = 4096 * 2048 + 5 * B
    codes, pc, scales, ps = _inputs(R, 4, numel, B, 31, random_bytes=True)
    cl = [codes[r * pc:(r + 1) * pc] for r in range(R)]
    sl = [scales[r * ps:(r + 1) * ps] for r in range(R)]
    co, so, _ = oracle_par.dequant_reduce_requant(cl, sl, 4, numel, B, 4)
    cd, sd = dev(codes), dev(scales)
    for k0, kl in ((777 * B, 1953 * B), (0, numel)):
        sc, ss, kc, ks = z.dequant_reduce_requant_split(cd, sd, R, 4, numel, B, k0, kl, 4)
        torch.cuda.synchronize()
        c0, c1 = k0 // 2, (k0 + kl) // 2
        assert_bits_equal(kc.cpu().numpy(), co[c0:c1], "keep codes")
        assert_bits_equal(ks.cpu().numpy(), so[k0 // B:(k0 + kl) // B], "keep scales")
        if kl < numel:
            assert_bits_equal(sc.cpu().numpy(), np.concatenate([co[:c0], co[c1:]]), "send codes")
            assert_bits_equal(ss.cpu().numpy(), np.concatenate([so[:k0 // B], so[(k0 + kl) // B:]]), "send scales")
        else:
            assert sc is None and ss is None
