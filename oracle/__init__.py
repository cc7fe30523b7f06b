"""CPU oracle of the ZeRO++ block-quantization codec (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library
(``block_quantization_codec_amd``) never does, and shares no code with it.

The arithmetic lives in ``zpp_oracle.c`` (plain scalar C, built with the
host compiler, no fused multiply-add); this module builds it, loads it with
ctypes and wraps it for numpy arrays. bfloat16 arrays are ``numpy.uint16``
bit patterns. See the C file's header for the passages each step follows
and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zpp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
          "-mfpmath=sse", "-msse2", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        for name, args in {
            "oracle_quantize_f32": [P, I64, I32, I32, P, P],
            "oracle_quantize_bf16": [P, I64, I32, I32, P, P],
            "oracle_dequantize_f32": [P, P, I32, I64, I32, P],
            "oracle_dequantize_bf16": [P, P, I32, I64, I32, P],
            "oracle_reorder_slices": [P, P, I64, I32, I32],
            "oracle_dequant_sum": [P, I64, P, I64, I32, I32, I64, I32, P],
            "oracle_dequant_reduce_requant": [P, I64, P, I64, I32, I32, I64, I32, P, P, I32, P],
            "oracle_dequant_average": [P, I64, P, I64, I32, I32, I64, I32, I32, P],
        }.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        for name in ("oracle_bf16_round_array", "oracle_bf16_decode_array"):
            f = getattr(L, name)
            f.argtypes = [P, I64, P]
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle rejected arguments of {what} (code {rc})")


def codes_nbytes(numel: int, bits: int) -> int:
    return numel * bits // 8


def _need(have: int, need: int, what: str) -> None:
    """The C routines read as much as numel implies: shorter arrays are refused here."""
    if have < need:
        raise ValueError(f"{what} holds {have} items, the call needs {need}")


def quantize(x: np.ndarray, block: int, bits: int):
    """Block-quantize ``x`` (uint16 bf16 bits or float32). Returns (codes uint8, scales float32)."""
    x = np.ascontiguousarray(x)
    n = x.size
    codes = np.zeros(codes_nbytes(n, bits), dtype=np.uint8)
    scales = np.zeros(n // block if block else 0, dtype=np.float32)
    if x.dtype == np.uint16:
        rc = lib().oracle_quantize_bf16(_ptr(x), n, block, bits, _ptr(codes), _ptr(scales))
    elif x.dtype == np.float32:
        rc = lib().oracle_quantize_f32(_ptr(x), n, block, bits, _ptr(codes), _ptr(scales))
    else:
        raise TypeError("quantize takes bf16 bit patterns (uint16) or float32")
    _check(rc, "quantize")
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, bits: int, numel: int, block: int,
               out: str = "f32") -> np.ndarray:
    """Dequantize to float32 (``out='f32'``) or bf16 bit patterns (``out='bf16'``)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    if block > 0:
        _need(codes.size, codes_nbytes(numel, bits), "codes")
        _need(scales.size, numel // block, "scales")
    if out == "f32":
        y = np.empty(numel, dtype=np.float32)
        rc = lib().oracle_dequantize_f32(_ptr(codes), _ptr(scales), bits, numel, block, _ptr(y))
    elif out == "bf16":
        y = np.empty(numel, dtype=np.uint16)
        rc = lib().oracle_dequantize_bf16(_ptr(codes), _ptr(scales), bits, numel, block, _ptr(y))
    else:
        raise ValueError(out)
    _check(rc, "dequantize")
    return y


def reorder_slices(buf: np.ndarray, n_nodes: int, gpus_per_node: int) -> np.ndarray:
    """Reorder the N = n_nodes*gpus_per_node equal slices of ``buf`` (any dtype)."""
    buf = np.ascontiguousarray(buf)
    n_slices = n_nodes * gpus_per_node
    if buf.nbytes % n_slices:
        raise ValueError("buffer does not split into equal slices")
    out = np.empty_like(buf)
    rc = lib().oracle_reorder_slices(_ptr(buf), _ptr(out), buf.nbytes // n_slices, n_nodes, gpus_per_node)
    _check(rc, "reorder")
    return out


def reorder_permutation(n_nodes: int, gpus_per_node: int) -> list[int]:
    """Source slice index for each output slice position, read off the C oracle."""
    n = n_nodes * gpus_per_node
    src = np.arange(n, dtype=np.int64)
    return [int(v) for v in reorder_slices(src, n_nodes, gpus_per_node)]


def dequant_sum(codes_list, scales_list, bits: int, numel: int, block: int) -> np.ndarray:
    """Sum of the inputs' dequantized values, in input order (binary32)."""
    codes = np.stack([np.ascontiguousarray(c, dtype=np.uint8) for c in codes_list])
    scales = np.stack([np.ascontiguousarray(s, dtype=np.float32) for s in scales_list])
    if block > 0:
        _need(codes.shape[1], codes_nbytes(numel, bits), "each input's codes")
        _need(scales.shape[1], numel // block, "each input's scales")
    out = np.empty(numel, dtype=np.float32)
    rc = lib().oracle_dequant_sum(_ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1],
                                  len(codes_list), bits, numel, block, _ptr(out))
    _check(rc, "dequant_sum")
    return out


def dequant_reduce_requant(codes_list, scales_list, bits_in: int, numel: int, block: int,
                           bits_out: int = 0):
    """Fused hop step. Returns (codes_out, scales_out, sum_f32); codes/scales are None
    when ``bits_out == 0``."""
    codes = np.stack([np.ascontiguousarray(c, dtype=np.uint8) for c in codes_list])
    scales = np.stack([np.ascontiguousarray(s, dtype=np.float32) for s in scales_list])
    if block > 0:
        _need(codes.shape[1], codes_nbytes(numel, bits_in), "each input's codes")
        _need(scales.shape[1], numel // block, "each input's scales")
    total = np.empty(numel, dtype=np.float32)
    co = so = None
    if bits_out:
        co = np.zeros(codes_nbytes(numel, bits_out), dtype=np.uint8)
        so = np.zeros(numel // block, dtype=np.float32)
    rc = lib().oracle_dequant_reduce_requant(
        _ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1], len(codes_list), bits_in,
        numel, block, _ptr(co), _ptr(so), bits_out, _ptr(total))
    _check(rc, "dequant_reduce_requant")
    return co, so, total


def dequant_average(codes_list, scales_list, bits: int, numel: int, block: int, divisor: int) -> np.ndarray:
    """The input-order binary32 sum divided by ``divisor`` (the number of GPUs
    that contributed), one correctly rounded division per element."""
    codes = np.stack([np.ascontiguousarray(c, dtype=np.uint8) for c in codes_list])
    scales = np.stack([np.ascontiguousarray(s, dtype=np.float32) for s in scales_list])
    if block > 0:
        _need(codes.shape[1], codes_nbytes(numel, bits), "each input's codes")
        _need(scales.shape[1], numel // block, "each input's scales")
    out = np.empty(numel, dtype=np.float32)
    rc = lib().oracle_dequant_average(_ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1],
                                      len(codes_list), bits, numel, block, divisor, _ptr(out))
    _check(rc, "dequant_average")
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.size, dtype=np.uint16)
    lib().oracle_bf16_round_array(_ptr(x), x.size, _ptr(y))
    return y


def bf16_decode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.empty(x.size, dtype=np.float32)
    lib().oracle_bf16_decode_array(_ptr(x), x.size, _ptr(y))
    return y
