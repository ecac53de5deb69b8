"""MI355X ternary rotated-basis linear y = W(Rx): thin Python binding of libtb.so.

Every computation runs in the HIP kernels of libtb.so; this module only checks
tensor arguments and marshals pointers, sizes and the current HIP stream into
the C ABI declared in include/tb.h.  PyTorch provides device memory and
streams.  There is no fallback: if libtb.so is missing or cannot be loaded,
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtb.so")

TB_PACK_2BIT, TB_PACK_BASE3 = 0, 1
TB_F32, TB_F16, TB_BF16 = 0, 1, 2
TB_GEMV_MAX_BATCH = 32   # tb_gemv: one pass over the weights at any batch up to this
TB_GEMV_KERNEL_BATCH = 8  # tb_linear above this: chunks of 8 rows, each re-streaming the weights
PACKINGS = {"2bit": TB_PACK_2BIT, "base3": TB_PACK_BASE3}

EXPORTS = ("tb_packed_row_bytes", "tb_pack_2bit", "tb_pack_base3", "tb_unpack", "tb_fwht_rotate",
           "tb_gemv", "tb_linear", "tb_gemm", "tb_status_string", "tb_last_hip_error")

_VP, _I64, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGNATURES = {
    "tb_packed_row_bytes": (_I64, [_INT, _I64]),
    "tb_pack_2bit": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP]),
    "tb_pack_base3": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP]),
    "tb_unpack": (_INT, [_INT, _VP, _I64, _I64, _VP, _VP, _VP]),
    "tb_fwht_rotate": (_INT, [_VP, _INT, _VP, _INT, _I64, _I64, _VP, _VP]),
    "tb_gemv": (_INT, [_INT, _VP, _VP, _VP, _INT, _VP, _I64, _I64, _I64, _VP]),
    "tb_linear": (_INT, [_INT, _VP, _VP, _VP, _INT, _VP, _VP, _I64, _I64, _I64, _VP]),
    "tb_gemm": (_INT, [_INT, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _VP]),
    "tb_status_string": (ctypes.c_char_p, [_INT]),
    "tb_last_hip_error": (ctypes.c_char_p, []),
}

_lib = None


class TBError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib_ = library()
        text = lib_.tb_status_string(status).decode()
        hip = lib_.tb_last_hip_error().decode()
        super().__init__(f"{fn} returned {status} ({text})" + (f": {hip}" if hip else ""))
        self.status = status


def library() -> ctypes.CDLL:
    """Load libtb.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with fwht_rotation_sqrt_amd.build.build()")
        lib_ = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib_, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib_
    return _lib


def _stream(stream=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _check(t: torch.Tensor, name: str, dtypes) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _call(name: str, *args) -> None:
    st = getattr(library(), name)(*args)
    if st != 0:
        raise TBError(name, st)


def _packing(p) -> int:
    return PACKINGS[p] if isinstance(p, str) else int(p)


_ACT_DT = {torch.float32: TB_F32, torch.float16: TB_F16, torch.bfloat16: TB_BF16}
_ACT_TORCH = {TB_F32: torch.float32, TB_F16: torch.float16}


def tb_packed_row_bytes(packing, k: int) -> int:
    return int(library().tb_packed_row_bytes(_packing(packing), int(k)))


def _pack(name, packing, trits, packed, bad_count, stream):
    _check(trits, "trits", (torch.int8,))
    n, k = trits.shape
    rb = tb_packed_row_bytes(packing, k)
    if rb < 0:
        raise ValueError("K must be a positive multiple of 128")
    if packed is None:
        packed = torch.empty((n, rb), dtype=torch.uint8, device=trits.device)
    _check(packed, "packed", (torch.uint8,))
    if bad_count is not None:
        _check(bad_count, "bad_count", (torch.int32,))
    _call(name, _ptr(trits), n, k, _ptr(packed), _ptr(bad_count), _stream(stream))
    return packed


def tb_pack_2bit(trits, packed=None, bad_count=None, stream=None):
    """int8 [N][K] trits -> uint8 [N][K/4] 2-bit codes."""
    return _pack("tb_pack_2bit", TB_PACK_2BIT, trits, packed, bad_count, stream)


def tb_pack_base3(trits, packed=None, bad_count=None, stream=None):
    """int8 [N][K] trits -> uint8 [N][26*K/128] base-3 codes."""
    return _pack("tb_pack_base3", TB_PACK_BASE3, trits, packed, bad_count, stream)


def tb_unpack(packing, packed, k: int, trits=None, bad_count=None, stream=None):
    """Packed codes -> int8 [N][K] trits."""
    _check(packed, "packed", (torch.uint8,))
    n = packed.shape[0]
    if trits is None:
        trits = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    _check(trits, "trits", (torch.int8,))
    if bad_count is not None:
        _check(bad_count, "bad_count", (torch.int32,))
    _call("tb_unpack", _packing(packing), _ptr(packed), n, int(k), _ptr(trits), _ptr(bad_count),
          _stream(stream))
    return trits


def tb_fwht_rotate(x, sign_bits, out_dtype=torch.float32, out=None, stream=None):
    """[rows][K] activations -> R_K x as fp32 or fp16."""
    _check(x, "x", tuple(_ACT_DT))
    _check(sign_bits, "sign_bits", (torch.int32,))
    rows, k = x.shape
    if out is None:
        out = torch.empty((rows, k), dtype=out_dtype, device=x.device)
    _check(out, "out", (torch.float32, torch.float16))
    _call("tb_fwht_rotate", _ptr(x), _ACT_DT[x.dtype], _ptr(out), _ACT_DT[out.dtype], rows, k,
          _ptr(sign_bits), _stream(stream))
    return out


def tb_gemv(packing, packed, scales, xr, y=None, stream=None):
    """y[B][N] = packed ternary W (g128 fp16 scales) times rotated activations xr[B][K]."""
    _check(packed, "packed", (torch.uint8,))
    _check(scales, "scales", (torch.float16,))
    _check(xr, "xr", (torch.float32, torch.float16))
    b, k = xr.shape
    n = packed.shape[0]
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=xr.device)
    _check(y, "y", (torch.float32,))
    _call("tb_gemv", _packing(packing), _ptr(packed), _ptr(scales), _ptr(xr), _ACT_DT[xr.dtype],
          _ptr(y), b, n, k, _stream(stream))
    return y


def tb_linear(packing, packed, scales, x, sign_bits, y=None, stream=None):
    """y[B][N] = packed ternary W times R_K x, x[B][K] unrotated (rotation inside the call)."""
    _check(packed, "packed", (torch.uint8,))
    _check(scales, "scales", (torch.float16,))
    _check(x, "x", tuple(_ACT_DT))
    _check(sign_bits, "sign_bits", (torch.int32,))
    b, k = x.shape
    n = packed.shape[0]
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _check(y, "y", (torch.float32,))
    _call("tb_linear", _packing(packing), _ptr(packed), _ptr(scales), _ptr(x), _ACT_DT[x.dtype],
          _ptr(sign_bits), _ptr(y), b, n, k, _stream(stream))
    return y


def tb_gemm(packing, packed, scales, xr, y=None, stream=None):
    """Y[M][N] = X'[M][K] (fp16) times the packed ternary weights, fp32 out."""
    _check(packed, "packed", (torch.uint8,))
    _check(scales, "scales", (torch.float16,))
    _check(xr, "xr", (torch.float16,))
    m, k = xr.shape
    n = packed.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xr.device)
    _check(y, "y", (torch.float32,))
    _call("tb_gemm", _packing(packing), _ptr(packed), _ptr(scales), _ptr(xr), _ptr(y), m, n, k,
          _stream(stream))
    return y
