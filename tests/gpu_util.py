"""Helpers for the GPU parity tests: device transfers and canary-guarded outputs."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

GUARD = 256  # bytes of canary before and after every guarded output
CANARY = 0xA5


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantization_codec_amd  # noqa: F401  (fails loudly if libzpp.so is missing)


def dev(a: np.ndarray, dtype=None):
    """numpy -> device tensor (uint16 arrays become bfloat16)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def host(t) -> np.ndarray:
    """device tensor -> numpy (bfloat16 becomes uint16 bit patterns)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Guarded:
    """A device output buffer with canary bytes on both sides."""

    def __init__(self, nbytes: int, device="cuda"):
        self.nbytes = int(nbytes)
        self.raw = torch.full((self.nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device=device)

    @property
    def ptr(self) -> int:
        return self.raw.data_ptr() + GUARD

    def bytes(self) -> np.ndarray:
        return host(self.raw[GUARD:GUARD + self.nbytes])

    def as_np(self, dtype) -> np.ndarray:
        return self.bytes().view(dtype)

    def untouched(self) -> bool:
        r = host(self.raw)
        return bool(np.all(r[:GUARD] == CANARY) and np.all(r[GUARD + self.nbytes:] == CANARY))

    def all_canary(self) -> bool:
        return bool(np.all(host(self.raw) == CANARY))


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype.itemsize == 4:
        g, w = got.view(np.uint32), want.view(np.uint32)
    elif got.dtype.itemsize == 2:
        g, w = got.view(np.uint16), want.view(np.uint16)
    else:
        g, w = got.view(np.uint8), want.view(np.uint8)
    bad = np.nonzero(g != w)[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at {i.tolist()}: "
                             f"got {g[i].tolist()} want {w[i].tolist()}")


def assert_within_scale(got: np.ndarray, want: np.ndarray, scale_per_elem: np.ndarray, what: str,
                        rel: float = 1e-5):
    """|got - want| <= rel * block scale, elementwise (the fp32 tolerance of the codec)."""
    d = np.abs(got.astype(np.float64) - want.astype(np.float64))
    lim = rel * scale_per_elem.astype(np.float64)
    bad = np.nonzero(d > lim)[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{what}: {bad.size} beyond {rel} x scale; first {i.tolist()}: "
                             f"got {got[i].tolist()} want {want[i].tolist()}")
