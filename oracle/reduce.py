"""Oracle for the W-way bf16 reduction (test infrastructure only).

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this module. It loads ``liboracle.so`` (plain C, built from
``arx_oracle.c`` by ``oracle/build.py``) and shares nothing with the HIP
library.

Page "arx.cu", reduction loop of ``arx_kernel``: out is the sum over ranks of
the partials, each bf16 widened to binary32, added in rank order 0..W-1 in
binary32, rounded once to bf16. Readings of the page: the accumulator starts
at -0.0f, NaN results become 0x7FC0, subnormals are kept, any n is allowed
(the page asks for n % 8 == 0) and elements at or past n are not written.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib() -> ctypes.CDLL:
    """Loads liboracle.so, building it first when it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        L.oracle_round_bf16.argtypes = [u32p, u16p, ctypes.c_size_t]
        L.oracle_round_bf16.restype = None
        L.oracle_widen_bf16.argtypes = [u16p, u32p, ctypes.c_size_t]
        L.oracle_widen_bf16.restype = None
        L.oracle_reduce.argtypes = [ctypes.POINTER(u16p), ctypes.c_int, ctypes.c_size_t, u16p]
        L.oracle_reduce.restype = None
        L.oracle_reduce_threads.argtypes = [ctypes.POINTER(u16p), ctypes.c_int, ctypes.c_size_t, u16p,
                                            ctypes.c_int]
        L.oracle_reduce_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p16(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def round_bf16(f32_bits: np.ndarray) -> np.ndarray:
    """binary32 bit patterns (uint32) -> bf16 bit patterns (uint16), RNE, NaN -> 0x7FC0."""
    a = np.ascontiguousarray(f32_bits, dtype=np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_round_bf16(_p32(a), _p16(out), a.size)
    return out


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> binary32 bit patterns (uint32), exact."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.uint32)
    lib().oracle_widen_bf16(_p16(a), _p32(out), a.size)
    return out


def reduce(parts, n: int = None, out: np.ndarray = None, threads: int = 1) -> np.ndarray:
    """Rank-ordered W-way reduction of bf16 partials.

    parts: sequence of W uint16 arrays (bf16 bits), parts[src] is rank src's
    partial. n: number of elements reduced (default: the shortest part).
    out: optional uint16 array of at least n elements; only out[:n] is
    written, the rest keeps its contents. threads: contiguous index ranges
    computed in parallel (same bits for any count).
    """
    arrs = [np.ascontiguousarray(p, dtype=np.uint16).reshape(-1) for p in parts]
    W = len(arrs)
    if W < 1:
        raise ValueError("need at least one partial")
    if n is None:
        n = min(a.size for a in arrs)
    if any(a.size < n for a in arrs):
        raise ValueError("a partial is shorter than n")
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    if out.dtype != np.uint16 or not out.flags.c_contiguous or out.size < n:
        raise ValueError("out must be a contiguous uint16 array of at least n elements")
    ptrs = (ctypes.POINTER(ctypes.c_uint16) * W)(*[_p16(a) for a in arrs])
    if threads <= 1:
        lib().oracle_reduce(ptrs, W, n, _p16(out))
    else:
        lib().oracle_reduce_threads(ptrs, W, n, _p16(out), int(threads))
    return out


def oneshot(in_bits: np.ndarray, recv, rank: int, W: int, n: int, par: int, out: np.ndarray = None):
    """One call of the one-shot path, reduction part (page "arx.cu", arx_kernel).

    in_bits: this rank's partial; recv[par][src] holds peer src's partial for
    parity par (entries at src == rank are ignored). Returns out, whose first
    n elements are the rank-ordered sum with this rank's partial at `rank`.
    """
    parts = [in_bits if src == rank else recv[par][src] for src in range(W)]
    return reduce(parts, n=n, out=out)
