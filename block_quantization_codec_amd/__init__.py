"""ZeRO++ block-quantization codec on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libzpp.so``, whose C ABI is ``include/zpp.h``. The
functions named like the C entry points take the same arguments in the same
order; a pointer argument may be a torch tensor (its ``data_ptr()`` is used)
or a plain integer address, and ``stream`` may be ``None`` (torch's current
stream), a ``torch.cuda.Stream`` or an integer ``hipStream_t``. They only
marshal arguments: every step runs in the library's HIP kernels, and a
non-OK status raises :class:`ZppError`.

The short helpers (:func:`quantize`, :func:`dequantize`, :func:`reorder`,
:func:`dequant_reduce_requant`, :func:`dequant_reduce_average`,
:func:`quantize_reordered`) allocate their outputs with torch on the
input's device and call the same entry points.

Importing the package fails with ``ImportError`` when ``libzpp.so`` has not
been built (``python block_quantization_codec_amd/_build.py``); there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzpp.so")

ZPP_OK = 0
ZPP_ERR_NULL = 1
ZPP_ERR_ARG = 2
ZPP_ERR_ALIGN = 3
ZPP_ERR_UNSUPPORTED = 4
ZPP_ERR_LAUNCH = 5
ZPP_ERR_OVERLAP = 6
ZPP_ERR_POINTER = 7

ZPP_BF16 = 1
ZPP_FP32 = 2

ZPP_MIN_BLOCK = 32
ZPP_MAX_BLOCK = 4096
ZPP_MAX_INPUTS = 4096
ZPP_MAX_DIVISOR = 1 << 24
ZPP_MAX_NUMEL = 1 << 40

EXPORTED = ("zpp_quantize_blocks", "zpp_quantize_reordered", "zpp_dequantize_blocks", "zpp_reorder_slices",
            "zpp_dequant_reduce_requant", "zpp_dequant_reduce_requant_split", "zpp_dequant_reduce_average",
            "zpp_set_pointer_checks", "zpp_status_string", "zpp_abi_version")


class ZppError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        super().__init__(f"{func}: {_lib.zpp_status_string(status).decode()}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: the codec runs only in its HIP library; build it with "
            "`python block_quantization_codec_amd/_build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sig = {
        "zpp_quantize_blocks": [P, I32, I64, I32, I32, P, P, P],
        "zpp_quantize_reordered": [P, I32, I64, I32, I32, I32, I32, I32, I32, P, P, P],
        "zpp_dequantize_blocks": [P, P, I32, I64, I32, P, I32, P],
        "zpp_reorder_slices": [P, P, I64, I32, I32, P],
        "zpp_dequant_reduce_requant": [P, I64, P, I64, I32, I32, I64, I32, P, P, I32, P, P],
        "zpp_dequant_reduce_requant_split": [P, I64, P, I64, I32, I32, I64, I32, I64, I64, P, P, P, P, I32, P],
        "zpp_dequant_reduce_average": [P, I64, P, I64, I32, I32, I64, I32, I32, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.zpp_set_pointer_checks.argtypes = [ctypes.c_int32]
    lib.zpp_set_pointer_checks.restype = ctypes.c_int32
    lib.zpp_status_string.argtypes = [ctypes.c_int]
    lib.zpp_status_string.restype = ctypes.c_char_p
    lib.zpp_abi_version.argtypes = []
    lib.zpp_abi_version.restype = ctypes.c_int32
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    """The loaded ``libzpp.so``."""
    return _lib


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name: str, *args) -> None:
    status = getattr(_lib, name)(*args)
    if status != ZPP_OK:
        raise ZppError(status, name)


# ---- the C entry points, same names and argument order ----------------------

def zpp_quantize_blocks(x, x_dtype, numel, block, bits, codes, scales, stream=None) -> None:
    _call("zpp_quantize_blocks", _ptr(x), x_dtype, numel, block, bits, _ptr(codes), _ptr(scales),
          _stream(stream))


def zpp_quantize_reordered(x, x_dtype, slice_elems, n_nodes, gpus_per_node, first_slice, n_slices, block, bits,
                           codes, scales, stream=None) -> None:
    _call("zpp_quantize_reordered", _ptr(x), x_dtype, slice_elems, n_nodes, gpus_per_node, first_slice, n_slices,
          block, bits, _ptr(codes), _ptr(scales), _stream(stream))


def zpp_dequantize_blocks(codes, scales, bits, numel, block, y, y_dtype, stream=None) -> None:
    _call("zpp_dequantize_blocks", _ptr(codes), _ptr(scales), bits, numel, block, _ptr(y), y_dtype,
          _stream(stream))


def zpp_reorder_slices(inp, out, slice_bytes, n_nodes, gpus_per_node, stream=None) -> None:
    _call("zpp_reorder_slices", _ptr(inp), _ptr(out), slice_bytes, n_nodes, gpus_per_node, _stream(stream))


def zpp_dequant_reduce_requant(codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs, bits_in,
                               numel, block, codes_out, scales_out, bits_out, sum_out, stream=None) -> None:
    _call("zpp_dequant_reduce_requant", _ptr(codes_in), codes_stride_bytes, _ptr(scales_in), scales_stride,
          n_inputs, bits_in, numel, block, _ptr(codes_out), _ptr(scales_out), bits_out, _ptr(sum_out),
          _stream(stream))


def zpp_dequant_reduce_requant_split(codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs, bits_in,
                                     numel, block, keep_begin, keep_elems, codes_send, scales_send, codes_keep,
                                     scales_keep, bits_out, stream=None) -> None:
    _call("zpp_dequant_reduce_requant_split", _ptr(codes_in), codes_stride_bytes, _ptr(scales_in), scales_stride,
          n_inputs, bits_in, numel, block, keep_begin, keep_elems, _ptr(codes_send), _ptr(scales_send),
          _ptr(codes_keep), _ptr(scales_keep), bits_out, _stream(stream))


def zpp_dequant_reduce_average(codes_in, codes_stride_bytes, scales_in, scales_stride, n_inputs, bits_in, numel,
                               block, divisor, avg_out, stream=None) -> None:
    _call("zpp_dequant_reduce_average", _ptr(codes_in), codes_stride_bytes, _ptr(scales_in), scales_stride,
          n_inputs, bits_in, numel, block, divisor, _ptr(avg_out), _stream(stream))


def zpp_set_pointer_checks(enabled: bool) -> bool:
    """Switch the library's HIP-runtime pointer and range checks on or off for
    the process (see include/zpp.h); returns the previous setting."""
    return bool(_lib.zpp_set_pointer_checks(1 if enabled else 0))


def zpp_status_string(status: int) -> str:
    return _lib.zpp_status_string(status).decode()


def zpp_abi_version() -> int:
    return int(_lib.zpp_abi_version())


# ---- allocating helpers ------------------------------------------------------

def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return ZPP_BF16
    if t.dtype == torch.float32:
        return ZPP_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32 expected")


def _need_contiguous(**tensors) -> None:
    """The kernels read flat buffers from data_ptr(): a strided view would be misread."""
    for name, t in tensors.items():
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def quantize(x, block: int, bits: int, stream=None):
    """Block-quantize a contiguous bf16/fp32 device tensor. Returns (codes uint8, scales fp32)."""
    import torch

    _need_contiguous(x=x)
    n = x.numel()
    codes = torch.empty(n * bits // 8, dtype=torch.uint8, device=x.device)
    scales = torch.empty(n // block, dtype=torch.float32, device=x.device)
    zpp_quantize_blocks(x, _dtype_code(x), n, block, bits, codes, scales, stream)
    return codes, scales


def quantize_reordered(x, n_nodes: int, gpus_per_node: int, block: int, bits: int, first_slice: int = 0,
                       n_slices: int | None = None, stream=None):
    """Quantize the tensor-slice reordered view of contiguous x (N equal slices)
    without writing the reordered tensor. Returns (codes, scales) of output slices
    [first_slice, first_slice + n_slices)."""
    import torch

    _need_contiguous(x=x)
    n = n_nodes * gpus_per_node
    if x.numel() % n:
        raise ValueError("tensor does not split into equal slices")
    slice_elems = x.numel() // n
    n_slices = n - first_slice if n_slices is None else n_slices
    out = slice_elems * n_slices
    codes = torch.empty(out * bits // 8, dtype=torch.uint8, device=x.device)
    scales = torch.empty(out // block, dtype=torch.float32, device=x.device)
    zpp_quantize_reordered(x, _dtype_code(x), slice_elems, n_nodes, gpus_per_node, first_slice, n_slices, block,
                           bits, codes, scales, stream)
    return codes, scales


def dequantize(codes, scales, bits: int, numel: int, block: int, dtype=None, stream=None):
    """Rebuild ``numel`` values (bf16 by default, or fp32) from codes and scales."""
    import torch

    _need_contiguous(codes=codes, scales=scales)
    dtype = dtype or torch.bfloat16
    y = torch.empty(numel, dtype=dtype, device=codes.device)
    zpp_dequantize_blocks(codes, scales, bits, numel, block, y, _dtype_code(y), stream)
    return y


def reorder(t, n_nodes: int, gpus_per_node: int, stream=None):
    """Reorder the n_nodes*gpus_per_node equal slices of a contiguous device tensor."""
    import torch

    _need_contiguous(t=t)
    n = n_nodes * gpus_per_node
    nbytes = t.numel() * t.element_size()
    if nbytes % n:
        raise ValueError("tensor does not split into equal slices")
    out = torch.empty_like(t)
    zpp_reorder_slices(t, out, nbytes // n, n_nodes, gpus_per_node, stream)
    return out


def dequant_reduce_requant(codes_in, scales_in, n_inputs: int, bits_in: int, numel: int, block: int,
                           bits_out: int = 0, want_sum: bool = True, codes_stride_bytes: int | None = None,
                           scales_stride: int | None = None, stream=None):
    """Sum ``n_inputs`` quantized pieces laid side by side (strides default to one
    piece) and optionally requantize. Returns (codes_out, scales_out, sum_out),
    with None for outputs not requested."""
    import torch

    _need_contiguous(codes_in=codes_in, scales_in=scales_in)
    dev = codes_in.device
    cs = codes_stride_bytes if codes_stride_bytes is not None else numel * bits_in // 8
    ss = scales_stride if scales_stride is not None else numel // block
    co = so = su = None
    if bits_out:
        co = torch.empty(numel * bits_out // 8, dtype=torch.uint8, device=dev)
        so = torch.empty(numel // block, dtype=torch.float32, device=dev)
    if want_sum:
        su = torch.empty(numel, dtype=torch.float32, device=dev)
    zpp_dequant_reduce_requant(codes_in, cs, scales_in, ss, n_inputs, bits_in, numel, block, co, so,
                               bits_out, su, stream)
    return co, so, su


def dequant_reduce_requant_split(codes_in, scales_in, n_inputs: int, bits_in: int, numel: int, block: int,
                                 keep_begin: int, keep_elems: int, bits_out: int,
                                 codes_stride_bytes: int | None = None, scales_stride: int | None = None,
                                 stream=None):
    """The requantized sum of ``n_inputs`` pieces split in one pass: elements
    [keep_begin, keep_begin + keep_elems) (whole blocks) to the kept pair, all
    others, in order, to the send pair. Returns (send_codes, send_scales,
    keep_codes, keep_scales), with None for an empty pair."""
    import torch

    _need_contiguous(codes_in=codes_in, scales_in=scales_in)
    dev = codes_in.device
    cs = codes_stride_bytes if codes_stride_bytes is not None else numel * bits_in // 8
    ss = scales_stride if scales_stride is not None else numel // block
    send = numel - keep_elems
    sc = torch.empty(send * bits_out // 8, dtype=torch.uint8, device=dev) if send > 0 else None
    sS = torch.empty(send // block, dtype=torch.float32, device=dev) if send > 0 else None
    kc = torch.empty(keep_elems * bits_out // 8, dtype=torch.uint8, device=dev) if keep_elems > 0 else None
    kS = torch.empty(keep_elems // block, dtype=torch.float32, device=dev) if keep_elems > 0 else None
    zpp_dequant_reduce_requant_split(codes_in, cs, scales_in, ss, n_inputs, bits_in, numel, block, keep_begin,
                                     keep_elems, sc, sS, kc, kS, bits_out, stream)
    return sc, sS, kc, kS


def dequant_reduce_average(codes_in, scales_in, n_inputs: int, bits_in: int, numel: int, block: int, divisor: int,
                           codes_stride_bytes: int | None = None, scales_stride: int | None = None, stream=None):
    """Sum ``n_inputs`` quantized pieces laid side by side and divide by ``divisor``
    (the number of contributing GPUs). Returns the fp32 average."""
    import torch

    _need_contiguous(codes_in=codes_in, scales_in=scales_in)
    cs = codes_stride_bytes if codes_stride_bytes is not None else numel * bits_in // 8
    ss = scales_stride if scales_stride is not None else numel // block
    avg = torch.empty(numel, dtype=torch.float32, device=codes_in.device)
    zpp_dequant_reduce_average(codes_in, cs, scales_in, ss, n_inputs, bits_in, numel, block, divisor, avg, stream)
    return avg
