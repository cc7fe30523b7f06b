"""GPU parity at the full workload sizes, in the launch shapes the benchmark uses.

Every output of every workload is compared with the oracle, bit for bit: the
4096x4096 weight, the 8-rank 2x4 chain, the 64-shard layer, the 500M-element
bucket at 32x8 (reorder, unfused and fused int4 quantize, the whole hop-1
chunk, the hop-2 slice and its average) and the 855M-element GQA layer
(int8 codes, scales and bf16 round trip of the weight; int4 codes, scales
and binary32 round trip of the gradient). At the two largest sizes the
oracle runs over independent block ranges on a thread pool
(tests/oracle_par.py), which gives the same bytes as one call. Inputs come
from the seeded generators; inputs the oracle needs in quantized form (peer
contributions) are quantized by the oracle, never by the GPU.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import oracle_par
import synth
from gpu_util import assert_bits_equal, assert_within_scale, dev, host, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _z():
    import block_quantization_codec_amd as z
    return z


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# --------------------------------------------------------------------------
# qwZ: 4096x4096 weight, int8, block 256 (complete comparison)
# --------------------------------------------------------------------------

def test_qwz_int8_4096x4096_round_trip():
    z = _z()
    w = synth.QWZ_INT8_4096
    _say(f"generate {w.name}")
    x = w.weight()
    xd = dev(x)
    codes, scales = z.quantize(xd, w.block, w.bits)
    y = z.dequantize(codes, scales, w.bits, x.size, w.block, dtype=torch.bfloat16)
    y32 = z.dequantize(codes, scales, w.bits, x.size, w.block, dtype=torch.float32)
    torch.cuda.synchronize()
    c_np, s_np = host(codes), host(scales)
    want_c, want_s = oracle.quantize(x, w.block, w.bits)
    assert_bits_equal(s_np, want_s, "scales")
    assert_bits_equal(c_np, want_c, "codes")
    assert_bits_equal(host(y), oracle.dequantize(want_c, want_s, 8, x.size, w.block, out="bf16"), "bf16")
    want32 = oracle.dequantize(want_c, want_s, 8, x.size, w.block, out="f32")
    assert_within_scale(host(y32), want32, np.repeat(want_s, w.block), "fp32 within 1e-5 s")
    # block quantization beats one global scale on this tensor (QWZ's precision claim, ratio reported)
    xv = oracle.bf16_decode(x).astype(np.float64)
    gc, gs = oracle.quantize(x, x.size, 8)
    e_blk = np.sqrt(np.mean((xv - want32) ** 2))
    e_glb = np.sqrt(np.mean((xv - oracle.dequantize(gc, gs, 8, x.size, x.size)) ** 2))
    _say(f"RMS error global/block = {e_glb / e_blk:.2f}")
    assert e_blk < e_glb


# --------------------------------------------------------------------------
# qgZ 2 nodes x 4 GPUs, 8 x 16,000,000, int4 block 128 (complete comparison)
# --------------------------------------------------------------------------

def test_qgz_int4_2x4_full_chain():
    z = _z()
    c = synth.QGZ_INT4_2x4
    n, g, N, B = c.n_nodes, c.gpus_per_node, c.n_ranks, c.block
    P, S, C = c.padded, c.slice_len, c.chunk_len
    _say(f"generate {c.name}")
    bufs = [c.bucket(r) for r in range(N)]
    grads = dev(np.concatenate(bufs))                       # [N][P] bf16
    reord = torch.empty_like(grads)
    for r in range(N):                                      # each rank reorders its bucket
        z.zpp_reorder_slices(grads[r * P:], reord[r * P:], S * 2, n, g)
    codes, scales = z.quantize(reord, B, 4)                 # one-shot quantize, all ranks
    # hop 1, one call per node: element-wise over the node's g buckets, which is
    # every local rank's hop-1 share side by side (rank (a, j) owns chunk j)
    h1c = torch.empty(n * P // 2, dtype=torch.uint8, device="cuda")
    h1s = torch.empty(n * P // B, dtype=torch.float32, device="cuda")
    for a in range(n):
        z.zpp_dequant_reduce_requant(codes[a * g * P // 2:], P // 2, scales[a * g * P // B:], P // B, g, 4, P, B,
                                     h1c[a * P // 2:], h1s[a * P // B:], 4, None)
    # hop 2, one call: element p of the sum over nodes lands on rank (k, j) for
    # p in chunk j, sub-chunk k
    final = torch.empty(P, dtype=torch.float32, device="cuda")
    z.zpp_dequant_reduce_requant(h1c, P // 2, h1s, P // B, n, 4, P, B, None, None, 0, final)
    # one GPU's share, as launched alone: rank 7's hop 1 (chunk 3 of ranks 4..7)
    a, j = 1, 3
    one_c = torch.empty(C // 2, dtype=torch.uint8, device="cuda")
    one_s = torch.empty(C // B, dtype=torch.float32, device="cuda")
    z.zpp_dequant_reduce_requant(codes[(a * g * P + j * C) // 2:], P // 2, scales[(a * g * P + j * C) // B:],
                                 P // B, g, 4, C, B, one_c, one_s, 4, None)
    torch.cuda.synchronize()

    _say("oracle chain")
    o_re = [oracle.reorder_slices(b, n, g) for b in bufs]
    assert_bits_equal(host(reord), np.concatenate(o_re), "reorder")
    oq = [oracle.quantize(b, B, 4) for b in o_re]
    assert_bits_equal(host(codes), np.concatenate([q[0] for q in oq]), "codes")
    assert_bits_equal(host(scales), np.concatenate([q[1] for q in oq]), "scales")
    o_h1 = []
    for a in range(n):
        co, so, _ = oracle.dequant_reduce_requant([oq[a * g + i][0] for i in range(g)],
                                                  [oq[a * g + i][1] for i in range(g)], 4, P, B, 4)
        o_h1.append((co, so))
    assert_bits_equal(host(h1c), np.concatenate([h[0] for h in o_h1]), "hop-1 codes")
    assert_bits_equal(host(h1s), np.concatenate([h[1] for h in o_h1]), "hop-1 scales")
    assert_bits_equal(host(one_c), o_h1[1][0][j * C // 2:(j + 1) * C // 2], "rank-7 share codes")
    assert_bits_equal(host(one_s), o_h1[1][1][j * C // B:(j + 1) * C // B], "rank-7 share scales")
    o_fin = oracle.dequant_sum([h[0] for h in o_h1], [h[1] for h in o_h1], 4, P, B)
    fin = host(final)
    smax = np.repeat(np.maximum(o_h1[0][1], o_h1[1][1]), B)
    assert_within_scale(fin, o_fin, smax, "final sum")
    assert_bits_equal(fin, o_fin, "final sum bits")
    # every rank ends with its own slice reduced over all 8 ranks (reduce-scatter)
    vals = [oracle.bf16_decode(b) for b in bufs]
    for k in range(n):
        for jj in range(g):
            r = k * g + jj
            exact = np.sum([v[r * S:(r + 1) * S].astype(np.float64) for v in vals], axis=0)
            pos = jj * C + k * S
            got = fin[pos:pos + S].astype(np.float64)
            assert np.max(np.abs(got - exact)) < 8 * 7 * 1e-3, r  # loose: several quantization steps


# --------------------------------------------------------------------------
# qwZ gather side: 64 int8 shards of a Llama-style layer, block 2048 (complete)
# --------------------------------------------------------------------------

def test_qwz_dequant_64_shards():
    z = _z()
    w = synth.QWZ_DEQUANT_64
    _say(f"generate {w.name}")
    x = w.weight()
    codes, scales = oracle.quantize(x, w.block, 8)  # each shard is 1,544 whole blocks
    assert (x.size // w.shards) % w.block == 0
    y = z.dequantize(dev(codes), dev(scales), 8, x.size, w.block, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bits_equal(host(y), oracle.dequantize(codes, scales, 8, x.size, w.block, out="bf16"), "bf16")


# --------------------------------------------------------------------------
# qgZ 32 nodes x 8 GPUs, one GPU's 500M-element bucket (rank 255), complete
# --------------------------------------------------------------------------

def test_qgz_int4_32x8_rank255_chain():
    z = _z()
    c = synth.QGZ_INT4_32x8
    n, g, B = c.n_nodes, c.gpus_per_node, c.block
    P, S, C = c.padded, c.slice_len, c.chunk_len
    node, local = n - 1, g - 1
    rank = node * g + local
    _say(f"generate {c.name} rank {rank}")
    bucket = c.bucket(rank)
    peers = [c.peer_chunk(i, local, node) for i in range(g - 1)]
    partials = [c.node_partial(a, node, local) for a in range(n - 1)]

    _say("oracle: reorder, quantize peers and partials")
    o_re = oracle.reorder_slices(bucket, n, g)
    own_chunk = o_re[local * C:(local + 1) * C]
    oq_own = oracle.quantize(own_chunk, B, 4)
    oq_peers = [oracle.quantize(p, B, 4) for p in peers]
    oq_parts = [oracle.quantize(p, B, 4) for p in partials]

    _say("gpu chain")
    bd = dev(bucket)
    reord = torch.empty_like(bd)
    z.zpp_reorder_slices(bd, reord, S * 2, n, g)
    codes, scales = z.quantize(reord, B, 4)
    # hop-1 receive buffer [g][C]: peers' chunks (oracle-quantized), own chunk last
    r1c = torch.empty(g * C // 2, dtype=torch.uint8, device="cuda")
    r1s = torch.empty(g * C // B, dtype=torch.float32, device="cuda")
    for i in range(g - 1):
        r1c[i * C // 2:(i + 1) * C // 2].copy_(dev(oq_peers[i][0]))
        r1s[i * C // B:(i + 1) * C // B].copy_(dev(oq_peers[i][1]))
    r1c[local * C // 2:].copy_(codes[local * C // 2:(local + 1) * C // 2])
    r1s[local * C // B:].copy_(scales[local * C // B:(local + 1) * C // B])
    h1c = torch.empty(C // 2, dtype=torch.uint8, device="cuda")
    h1s = torch.empty(C // B, dtype=torch.float32, device="cuda")
    z.zpp_dequant_reduce_requant(r1c, C // 2, r1s, C // B, g, 4, C, B, h1c, h1s, 4, None)
    # hop-2 receive buffer [n][S]: other nodes' partials, own sub-chunk `node` last
    r2c = torch.empty(n * S // 2, dtype=torch.uint8, device="cuda")
    r2s = torch.empty(n * S // B, dtype=torch.float32, device="cuda")
    for a in range(n - 1):
        r2c[a * S // 2:(a + 1) * S // 2].copy_(dev(oq_parts[a][0]))
        r2s[a * S // B:(a + 1) * S // B].copy_(dev(oq_parts[a][1]))
    r2c[node * S // 2:].copy_(h1c[node * S // 2:(node + 1) * S // 2])
    r2s[node * S // B:].copy_(h1s[node * S // B:(node + 1) * S // B])
    final = torch.empty(S, dtype=torch.float32, device="cuda")
    z.zpp_dequant_reduce_requant(r2c, S // 2, r2s, S // B, n, 4, S, B, None, None, 0, final)
    # the optimizer-ready shard: the same sum averaged over all n * g GPUs
    avg = torch.empty(S, dtype=torch.float32, device="cuda")
    z.zpp_dequant_reduce_average(r2c, S // 2, r2s, S // B, n, 4, S, B, n * g, avg)
    # the fused path as the benchmark launches it: chunks 0..6 and chunk 7
    fc = torch.empty(P // 2, dtype=torch.uint8, device="cuda")
    fs = torch.empty(P // B, dtype=torch.float32, device="cuda")
    z.zpp_quantize_reordered(bd, z.ZPP_BF16, S, n, g, 0, local * n, B, 4, fc, fs)
    z.zpp_quantize_reordered(bd, z.ZPP_BF16, S, n, g, local * n, n, B, 4, fc[local * C // 2:], fs[local * C // B:])
    torch.cuda.synchronize()

    _say("compare reorder (complete)")
    assert_bits_equal(host(reord), o_re, "reorder")
    del reord
    _say("compare quantize, unfused and fused (complete)")
    oc, os_ = oracle_par.quantize(o_re, B, 4)
    assert_bits_equal(oc[local * C // 2:(local + 1) * C // 2], oq_own[0], "oracle own chunk, two ways")
    assert_bits_equal(host(codes), oc, "codes")
    assert_bits_equal(host(scales), os_, "scales")
    assert_bits_equal(host(fc), oc, "fused reorder+quantize codes")
    assert_bits_equal(host(fs), os_, "fused reorder+quantize scales")
    del oc, os_
    _say("compare hop 1 (complete)")
    ins_c = [q[0] for q in oq_peers] + [oq_own[0]]
    ins_s = [q[1] for q in oq_peers] + [oq_own[1]]
    co, so, _ = oracle_par.dequant_reduce_requant(ins_c, ins_s, 4, C, B, 4)
    assert_bits_equal(host(h1c), co, "hop-1 codes")
    assert_bits_equal(host(h1s), so, "hop-1 scales")
    _say("compare hop 2 (complete slice)")
    own_sub = (co[node * S // 2:(node + 1) * S // 2], so[node * S // B:(node + 1) * S // B])
    o_fin = oracle.dequant_sum([q[0] for q in oq_parts] + [own_sub[0]], [q[1] for q in oq_parts] + [own_sub[1]],
                               4, S, B)
    fin = host(final)
    smax = np.repeat(np.max(np.stack([q[1] for q in oq_parts] + [own_sub[1]]), axis=0), B)
    assert_within_scale(fin, o_fin, smax, "hop-2 sum")
    assert_bits_equal(fin, o_fin, "hop-2 sum bits")
    o_avg = oracle.dequant_average([q[0] for q in oq_parts] + [own_sub[0]],
                                   [q[1] for q in oq_parts] + [own_sub[1]], 4, S, B, n * g)
    assert_bits_equal(host(avg), o_avg, "hop-2 average over 256 GPUs")
    real = c.real_in_slice(rank)
    assert real == 1_913_600 and not fin[real:].any(), "padding must reduce to zero"


# --------------------------------------------------------------------------
# 70B-scale GQA layer: int8 weight block 512, int4 gradient block 128, complete
# --------------------------------------------------------------------------

def test_gqa_layer_mixed_codec():
    z = _z()
    _say("generate GQA layer weight and gradient")
    W = synth.gqa_weight()
    G = synth.gqa_grad()
    n = W.size
    wd, gd = dev(W), dev(G)
    wc, ws = z.quantize(wd, 512, 8)
    wy = z.dequantize(wc, ws, 8, n, 512, dtype=torch.bfloat16)
    gc, gs = z.quantize(gd, 128, 4)
    gy = z.dequantize(gc, gs, 4, n, 128, dtype=torch.float32)
    torch.cuda.synchronize()
    _say("whole-output properties")
    # every int8 code in [-127, 127]; every block with a nonzero scale has a +-127 code
    q = wc.view(torch.int8)
    assert int(q.min()) >= -127 and int(q.max()) <= 127
    amax = q.view(-1, 512).abs().amax(dim=1)
    assert bool(((amax == 127) | (ws == 0)).all())
    # the rebuilt weight is within half a scale (+ binary32 and bf16 rounding) everywhere
    err = (wy.float() - wd.float()).abs().view(-1, 512)
    lim = ws.view(-1, 1) * (0.5 + 2.0 ** -15) + wy.float().abs().view(-1, 512) * 2.0 ** -8
    assert bool((err <= lim).all())
    del q, amax, err, lim, wd, gd

    _say("compare the weight's int8 codes, scales and bf16 round trip (complete)")
    oc, os_ = oracle_par.quantize(W, 512, 8)
    assert_bits_equal(host(ws), os_, "weight scales")
    assert_bits_equal(host(wc), oc, "weight codes")
    del wc
    assert_bits_equal(host(wy), oracle_par.dequantize(oc, os_, 8, n, 512, out="bf16"), "weight bf16")
    del wy, oc, os_, W
    _say("compare the gradient's int4 codes, scales and binary32 round trip (complete)")
    oc, os_ = oracle_par.quantize(G, 128, 4)
    assert_bits_equal(host(gs), os_, "grad scales")
    assert_bits_equal(host(gc), oc, "grad codes")
    want = oracle_par.dequantize(oc, os_, 4, n, 128, out="f32")
    got = host(gy)
    assert_within_scale(got, want, np.repeat(os_, 128), "grad fp32 within 1e-5 s")
    assert_bits_equal(got, want, "grad fp32 bits")
