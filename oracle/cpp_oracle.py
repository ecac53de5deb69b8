"""ctypes access to the plain C++ oracle (test infrastructure only).

``linear`` computes y = W_hat (R_K x) in float64 with plain loops (see
oracle/cpp/ternary_oracle.cpp for the passages it follows), its output rows
split over ``threads`` std::threads.  The library is built by
``oracle.cpp_build.build()`` (``__graft_entry__.build()`` calls it).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .cpp_build import LIB, SRC, build

_lib = None


def library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(SRC) > os.path.getmtime(LIB):
            build()  # missing, or older than its source
        lib = ctypes.CDLL(LIB)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.oracle_linear.restype = ctypes.c_int
        lib.oracle_linear.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_int]
        for name in ("oracle_pack", "oracle_unpack"):
            getattr(lib, name).restype = i64
            getattr(lib, name).argtypes = [ctypes.c_int, vp, i64, i64, vp]
        _lib = lib
    return _lib


def linear(packing: str, packed: np.ndarray, scales_bits: np.ndarray, x: np.ndarray,
           sign_bits: np.ndarray | None, threads: int = 1) -> np.ndarray:
    """float64 y [B][N]; x [B][K] unrotated (sign_bits given) or already rotated (None)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales_bits = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float64)
    b, k = x.shape
    n = packed.shape[0]
    y = np.empty((b, n), dtype=np.float64)
    sb = None if sign_bits is None else np.ascontiguousarray(sign_bits, dtype=np.uint32)
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    st = library().oracle_linear(0 if packing == "2bit" else 1, ptr(packed), ptr(scales_bits), ptr(x), ptr(sb),
                                 b, n, k, ptr(y), int(threads))
    if st != 0:
        raise ValueError(f"oracle_linear rejected the sizes (B={b}, N={n}, K={k})")
    return y


def pack(packing: str, trits: np.ndarray):
    """int8 [N][K] trits -> (uint8 packed [N][row bytes], invalid-trit count)."""
    t = np.ascontiguousarray(trits, dtype=np.int8)
    n, k = t.shape
    out = np.empty((n, k // 4 if packing == "2bit" else 26 * (k // 128)), dtype=np.uint8)
    bad = library().oracle_pack(0 if packing == "2bit" else 1, t.ctypes.data, n, k, out.ctypes.data)
    if bad < 0:
        raise ValueError(f"oracle_pack rejected the sizes (N={n}, K={k})")
    return out, int(bad)


def unpack(packing: str, packed: np.ndarray, k: int):
    """uint8 packed [N][row bytes] -> (int8 trits [N][K], invalid-code count)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    n = p.shape[0]
    out = np.empty((n, k), dtype=np.int8)
    bad = library().oracle_unpack(0 if packing == "2bit" else 1, p.ctypes.data, n, k, out.ctypes.data)
    if bad < 0:
        raise ValueError(f"oracle_unpack rejected the sizes (N={n}, K={k})")
    return out, int(bad)
