"""Argument errors that need the HIP runtime, on real device buffers.

Every entry point must return its status without launching anything: the
canary bytes around every output stay as they were. Covered here: ordinary
host memory passed as a device pointer (ZPP_ERR_POINTER), a buffer whose
byte range runs past its allocation (ZPP_ERR_ARG), misaligned pointers
(ZPP_ERR_ALIGN) and overlapping buffers (ZPP_ERR_OVERLAP). Pinned host
memory, which the GPU can address, is accepted as input and gives the same
result as device memory. A HIP error left pending by an unrelated earlier
call does not make a good call fail. Buffers carved from one allocation are
checked against it (a range that starts inside but runs past it is still
refused), and with the HIP-runtime pointer checks switched off the pure
argument checks still report.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import GUARD, Guarded, assert_bits_equal, dev, host, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _z():
    import block_quantization_codec_amd as z
    return z


def _expect_status(status, fn, *guards):
    z = _z()
    with pytest.raises(z.ZppError) as e:
        fn()
    assert e.value.status == status, z.zpp_status_string(e.value.status)
    torch.cuda.synchronize()
    for g in guards:
        assert g.all_canary(), "an output was written although the call failed"


def test_host_memory_is_rejected_everywhere():
    z = _z()
    n, B = 4096, 256
    host_buf = np.zeros(n * 4, np.uint8)  # ordinary pageable host memory
    hp = host_buf.ctypes.data
    x = dev(synth.small_bf16(n, (0, 501), 0.02))
    sin = torch.ones(2 * n // B, dtype=torch.float32, device="cuda")  # input scales
    gc, gs, gy = Guarded(n), Guarded(4 * n // B), Guarded(2 * n)
    P = z.ZPP_ERR_POINTER
    _expect_status(P, lambda: z.zpp_quantize_blocks(hp, z.ZPP_BF16, n, B, 8, gc.ptr, gs.ptr), gc, gs)
    _expect_status(P, lambda: z.zpp_quantize_blocks(x, z.ZPP_BF16, n, B, 8, hp, gs.ptr), gs)
    _expect_status(P, lambda: z.zpp_quantize_reordered(hp, z.ZPP_BF16, n // 4, 2, 2, 0, 4, B, 4, gc.ptr, gs.ptr),
                   gc, gs)
    _expect_status(P, lambda: z.zpp_dequantize_blocks(hp, sin, 8, n, B, gy.ptr, z.ZPP_BF16), gy)
    _expect_status(P, lambda: z.zpp_reorder_slices(hp, gy.ptr, n // 2, 2, 2), gy)
    _expect_status(P, lambda: z.zpp_dequant_reduce_requant(hp, 0, sin, 0, 2, 8, n, B, gc.ptr, gs.ptr, 8, None),
                   gc, gs)
    _expect_status(P, lambda: z.zpp_dequant_reduce_average(hp, 0, sin, 0, 2, 8, n, B, 2, gy.ptr), gy)


def test_range_past_the_allocation_is_rejected():
    """Hop reduction with a stride that carries input 1 a gigabyte past its
    allocation. The input is the highest of the buffers, so the claimed
    range cannot overlap an output and only the allocation check can fail."""
    z = _z()
    n, B = 1024, 256
    bufs = [Guarded(4096) for _ in range(3)]
    bufs.sort(key=lambda g: g.ptr)
    gc, gs, codes_in = bufs
    sin = torch.ones(2 * n // B, dtype=torch.float32, device="cuda")  # inputs may overlap each other
    _expect_status(z.ZPP_ERR_ARG,
                   lambda: z.zpp_dequant_reduce_requant(codes_in.ptr, 1 << 30, sin, 0, 2, 8, n, B, gc.ptr, gs.ptr,
                                                        8, None), gc, gs)


def test_misaligned_and_overlapping_buffers_are_rejected():
    z = _z()
    n, B = 4096, 256
    x = dev(synth.small_bf16(n, (0, 503), 0.02))
    gc, gs = Guarded(n + 64), Guarded(4 * n // B + 64)
    _expect_status(z.ZPP_ERR_ALIGN, lambda: z.zpp_quantize_blocks(x, z.ZPP_BF16, n, B, 8, gc.ptr + 8, gs.ptr),
                   gc, gs)
    _expect_status(z.ZPP_ERR_ALIGN, lambda: z.zpp_quantize_blocks(x, z.ZPP_BF16, n, B, 8, gc.ptr, gs.ptr + 2),
                   gc, gs)
    _expect_status(z.ZPP_ERR_OVERLAP, lambda: z.zpp_quantize_blocks(x, z.ZPP_BF16, n, B, 8, gc.ptr, gc.ptr + 64),
                   gc)
    _expect_status(z.ZPP_ERR_OVERLAP,
                   lambda: z.zpp_quantize_blocks(x, z.ZPP_BF16, n, B, 8, x.data_ptr(), gs.ptr), gs)
    assert GUARD >= 64


def test_pinned_host_input_is_accepted():
    z = _z()
    n, B = 1 << 16, 256
    xh = torch.from_numpy(synth.small_bf16(n, (0, 504), 0.02, 1e-3, 50.0)).view(torch.int16)
    pinned = torch.empty(n, dtype=torch.int16, pin_memory=True)
    pinned.copy_(xh)
    xd = pinned.cuda()
    c1 = torch.empty(n, dtype=torch.uint8, device="cuda")
    s1 = torch.empty(n // B, dtype=torch.float32, device="cuda")
    z.zpp_quantize_blocks(pinned.data_ptr(), z.ZPP_BF16, n, B, 8, c1, s1)
    c2, s2 = z.quantize(xd.view(torch.bfloat16), B, 8)
    torch.cuda.synchronize()
    assert_bits_equal(host(c1), host(c2), "codes from pinned host input")
    assert_bits_equal(host(s1), host(s2), "scales from pinned host input")


def test_pending_hip_error_does_not_fail_a_good_call():
    """An error an earlier, unrelated HIP call left pending in this thread
    (here: an attribute query for a device that does not exist) must not make
    a valid launch report ZPP_ERR_LAUNCH; the call clears it. The runtime is
    opened by the soname the library links, so it is the one already loaded."""
    import ctypes
    z = _z()
    n, B = 4096, 256
    x = synth.small_bf16(n, (0, 505), 0.02)
    xd = dev(x)
    c = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.empty(n // B, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so.7")
    value = ctypes.c_int(0)
    assert hip.hipDeviceGetAttribute(ctypes.byref(value), 0, 100000) != 0   # no device 100000
    assert hip.hipPeekAtLastError() != 0
    z.zpp_quantize_blocks(xd, z.ZPP_BF16, n, B, 8, c, s)   # raises ZppError if it reports a failure
    assert hip.hipPeekAtLastError() == 0
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize(x, B, 8)
    assert_bits_equal(host(c), oc, "codes after a pending error")
    assert_bits_equal(host(s), os_, "scales after a pending error")


def test_buffers_carved_from_one_allocation():
    """Input and outputs carved out of one device allocation, as torch's
    caching allocator hands them out: the allocation is looked up once and
    the later buffers inside it are accepted; the result matches the oracle
    and the bytes between the buffers stay untouched."""
    z = _z()
    n, B = 4096, 256
    x = synth.small_bf16(n, (0, 506), 0.02, 1e-3, 50.0)
    arena = torch.full((3 * 16384,), 0xA5, dtype=torch.uint8, device="cuda")
    arena[:2 * n].copy_(torch.from_numpy(x.view(np.uint8)).cuda())
    base = arena.data_ptr()
    z.zpp_quantize_blocks(base, z.ZPP_BF16, n, B, 8, base + 16384, base + 32768)
    torch.cuda.synchronize()
    a = host(arena)
    oc, os_ = oracle.quantize(x, B, 8)
    assert_bits_equal(a[16384:16384 + n], oc, "codes")
    assert_bits_equal(a[32768:32768 + 4 * n // B].view(np.float32), os_, "scales")
    assert np.all(a[2 * n:16384] == 0xA5) and np.all(a[16384 + n:32768] == 0xA5)
    assert np.all(a[32768 + 4 * n // B:] == 0xA5)


def test_range_starting_in_a_checked_allocation_but_running_past_it():
    """The codes are found inside their allocation; the scales start in the
    same allocation but their stride carries the second input a gigabyte past
    its end: still ZPP_ERR_ARG, nothing written."""
    z = _z()
    n, B = 1024, 256
    bufs = [Guarded(8192) for _ in range(3)]
    bufs.sort(key=lambda g: g.ptr)
    gc, gs, arena = bufs  # the inputs' allocation is the highest, so the claimed range overlaps no output
    _expect_status(z.ZPP_ERR_ARG,
                   lambda: z.zpp_dequant_reduce_requant(arena.ptr, 0, arena.ptr + 4096, 1 << 28, 2, 8, n, B, gc.ptr,
                                                        gs.ptr, 8, None), gc, gs)


def test_pointer_checks_switched_off():
    """With the HIP-runtime pointer checks off, valid calls give the same
    result and every pure argument check still reports; switched back on,
    host memory is refused again. (Only valid pointers are passed while the
    checks are off: an invalid one would reach the GPU.)"""
    z = _z()
    n, B = 4096, 256
    x = synth.small_bf16(n, (0, 507), 0.02, 1e-3, 50.0)
    xd = dev(x)
    gc, gs = Guarded(n + 64), Guarded(4 * n // B + 64)
    assert z.zpp_set_pointer_checks(False) is True
    try:
        c = torch.empty(n, dtype=torch.uint8, device="cuda")
        s = torch.empty(n // B, dtype=torch.float32, device="cuda")
        z.zpp_quantize_blocks(xd, z.ZPP_BF16, n, B, 8, c, s)
        torch.cuda.synchronize()
        oc, os_ = oracle.quantize(x, B, 8)
        assert_bits_equal(host(c), oc, "codes, checks off")
        assert_bits_equal(host(s), os_, "scales, checks off")
        _expect_status(z.ZPP_ERR_ALIGN, lambda: z.zpp_quantize_blocks(xd, z.ZPP_BF16, n, B, 8, gc.ptr + 8, gs.ptr),
                       gc, gs)
        _expect_status(z.ZPP_ERR_OVERLAP,
                       lambda: z.zpp_quantize_blocks(xd, z.ZPP_BF16, n, B, 8, gc.ptr, gc.ptr + 64), gc)
        _expect_status(z.ZPP_ERR_NULL, lambda: z.zpp_quantize_blocks(xd, z.ZPP_BF16, n, B, 8, None, gs.ptr), gs)
        assert z.zpp_set_pointer_checks(False) is False
    finally:
        z.zpp_set_pointer_checks(True)
    host_buf = np.zeros(2 * n, np.uint8)
    _expect_status(z.ZPP_ERR_POINTER,
                   lambda: z.zpp_quantize_blocks(host_buf.ctypes.data, z.ZPP_BF16, n, B, 8, gc.ptr, gs.ptr), gc, gs)
