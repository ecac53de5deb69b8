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
TB_STREAM_SINK_WORDS = 8192
TB_CHAIN_MAX = 8


class ChainLinear(ctypes.Structure):
    """tb_chain_linear: one linear of a tb_decode_chain call."""
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64)]
PACKINGS = {"2bit": TB_PACK_2BIT, "base3": TB_PACK_BASE3}

EXPORTS = ("tb_packed_row_bytes", "tb_pack_2bit", "tb_pack_base3", "tb_unpack", "tb_fwht_rotate",
           "tb_gemv", "tb_linear", "tb_linear_workspace_bytes", "tb_linear_ws", "tb_linear_noalloc", "tb_gemm",
           "tb_ternarize", "tb_decode_chain",
           "tb_stream_read", "tb_status_string", "tb_last_hip_error")

_VP, _I64, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGNATURES = {
    "tb_packed_row_bytes": (_I64, [_INT, _I64]),
    "tb_pack_2bit": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP]),
    "tb_pack_base3": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP]),
    "tb_unpack": (_INT, [_INT, _VP, _I64, _I64, _VP, _VP, _VP]),
    "tb_fwht_rotate": (_INT, [_VP, _INT, _VP, _INT, _I64, _I64, _VP, _VP]),
    "tb_gemv": (_INT, [_INT, _VP, _VP, _VP, _INT, _VP, _I64, _I64, _I64, _VP]),
    "tb_linear": (_INT, [_INT, _VP, _VP, _VP, _INT, _VP, _VP, _I64, _I64, _I64, _VP]),
    "tb_linear_workspace_bytes": (_I64, [_INT, _I64, _I64, _I64]),
    "tb_linear_ws": (_INT, [_INT, _VP, _VP, _VP, _INT, _VP, _VP, _I64, _I64, _I64, _VP, _I64, _VP]),
    "tb_linear_noalloc": (_INT, [_INT, _VP, _VP, _VP, _INT, _VP, _VP, _I64, _I64, _I64, _VP]),
    "tb_gemm": (_INT, [_INT, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _VP]),
    "tb_ternarize": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
    "tb_stream_read": (_INT, [_VP, _I64, _VP, _I64, _VP]),
    "tb_decode_chain": (_INT, [_INT, _VP, _INT, _VP, _INT, _VP, _I64, _VP, _I64, _INT, _VP]),
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


def _shape(t: torch.Tensor, name: str, want) -> None:
    """Exact shape check before any launch: the kernels size their reads and
    writes from the integer arguments, not from the tensors."""
    if tuple(t.shape) != tuple(int(w) for w in want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(w) for w in want)}")


def _rank2(t: torch.Tensor, name: str) -> None:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")


def _row_bytes(packing, k: int) -> int:
    rb = tb_packed_row_bytes(packing, k)
    if rb < 0:
        raise ValueError(f"K = {k} is not a positive multiple of 128 (or the packing is unknown)")
    return rb


def _weights(packing, packed, scales, k: int) -> int:
    """Check packed [N][row bytes] and scales [N][K/128]; return N."""
    _check(packed, "packed", (torch.uint8,))
    _check(scales, "scales", (torch.float16,))
    _rank2(packed, "packed")
    n = packed.shape[0]
    _shape(packed, "packed", (n, _row_bytes(packing, k)))
    _shape(scales, "scales", (n, k // 128))
    return n


def _signs(sign_bits: torch.Tensor, k: int) -> None:
    _check(sign_bits, "sign_bits", (torch.int32,))
    if sign_bits.dim() != 1 or sign_bits.numel() != k // 32:
        raise ValueError(f"sign_bits must hold K/32 = {k // 32} int32 words, got shape {tuple(sign_bits.shape)}")


def _count(bad_count) -> None:
    if bad_count is not None:
        _check(bad_count, "bad_count", (torch.int32,))
        if bad_count.numel() < 1:
            raise ValueError("bad_count must hold at least one int32")


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
    _rank2(trits, "trits")
    n, k = trits.shape
    rb = _row_bytes(packing, k)
    if packed is None:
        packed = torch.empty((n, rb), dtype=torch.uint8, device=trits.device)
    _check(packed, "packed", (torch.uint8,))
    _shape(packed, "packed", (n, rb))
    _count(bad_count)
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
    _rank2(packed, "packed")
    n, k = packed.shape[0], int(k)
    _shape(packed, "packed", (n, _row_bytes(packing, k)))
    if trits is None:
        trits = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    _check(trits, "trits", (torch.int8,))
    _shape(trits, "trits", (n, k))
    _count(bad_count)
    _call("tb_unpack", _packing(packing), _ptr(packed), n, int(k), _ptr(trits), _ptr(bad_count),
          _stream(stream))
    return trits


def tb_fwht_rotate(x, sign_bits, out_dtype=torch.float32, out=None, stream=None):
    """[rows][K] activations -> R_K x as fp32 or fp16."""
    _check(x, "x", tuple(_ACT_DT))
    _rank2(x, "x")
    rows, k = x.shape
    _signs(sign_bits, k)
    if out is None:
        out = torch.empty((rows, k), dtype=out_dtype, device=x.device)
    _check(out, "out", (torch.float32, torch.float16))
    _shape(out, "out", (rows, k))
    _call("tb_fwht_rotate", _ptr(x), _ACT_DT[x.dtype], _ptr(out), _ACT_DT[out.dtype], rows, k,
          _ptr(sign_bits), _stream(stream))
    return out


def tb_gemv(packing, packed, scales, xr, y=None, stream=None):
    """y[B][N] = packed ternary W (g128 fp16 scales) times rotated activations xr[B][K]."""
    _check(xr, "xr", (torch.float32, torch.float16))
    _rank2(xr, "xr")
    b, k = xr.shape
    n = _weights(packing, packed, scales, k)
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=xr.device)
    _check(y, "y", (torch.float32,))
    _shape(y, "y", (b, n))
    _call("tb_gemv", _packing(packing), _ptr(packed), _ptr(scales), _ptr(xr), _ACT_DT[xr.dtype],
          _ptr(y), b, n, k, _stream(stream))
    return y


def tb_linear(packing, packed, scales, x, sign_bits, y=None, stream=None):
    """y[B][N] = packed ternary W times R_K x, x[B][K] unrotated (rotation inside the call)."""
    _check(x, "x", tuple(_ACT_DT))
    _rank2(x, "x")
    b, k = x.shape
    n = _weights(packing, packed, scales, k)
    _signs(sign_bits, k)
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _check(y, "y", (torch.float32,))
    _shape(y, "y", (b, n))
    _call("tb_linear", _packing(packing), _ptr(packed), _ptr(scales), _ptr(x), _ACT_DT[x.dtype],
          _ptr(sign_bits), _ptr(y), b, n, k, _stream(stream))
    return y


def tb_linear_workspace_bytes(packing, b: int, n: int, k: int) -> int:
    return int(library().tb_linear_workspace_bytes(_packing(packing), int(b), int(n), int(k)))


def tb_linear_ws(packing, packed, scales, x, sign_bits, workspace=None, y=None, stream=None):
    """tb_linear with one pass over the weights at every batch; x' (batches from the crossover
    with the fused kernel on) or the partial sums of the parts of long base-3 rows (batch 1) go
    to ``workspace`` (a 16-byte aligned device tensor of at least tb_linear_workspace_bytes
    bytes)."""
    _check(x, "x", tuple(_ACT_DT))
    _rank2(x, "x")
    b, k = x.shape
    n = _weights(packing, packed, scales, k)
    _signs(sign_bits, k)
    need = tb_linear_workspace_bytes(packing, b, n, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _check(y, "y", (torch.float32,))
    _shape(y, "y", (b, n))
    _call("tb_linear_ws", _packing(packing), _ptr(packed), _ptr(scales), _ptr(x), _ACT_DT[x.dtype],
          _ptr(sign_bits), _ptr(y), b, n, k, _ptr(workspace), ws_bytes, _stream(stream))
    return y


def tb_linear_noalloc(packing, packed, scales, x, sign_bits, y, stream=None):
    """tb_linear_ws with x' in the library's static device scratch: no allocation anywhere
    (y must be given)."""
    _check(x, "x", tuple(_ACT_DT))
    _rank2(x, "x")
    b, k = x.shape
    n = _weights(packing, packed, scales, k)
    _signs(sign_bits, k)
    _check(y, "y", (torch.float32,))
    _shape(y, "y", (b, n))
    _call("tb_linear_noalloc", _packing(packing), _ptr(packed), _ptr(scales), _ptr(x), _ACT_DT[x.dtype],
          _ptr(sign_bits), _ptr(y), b, n, k, _stream(stream))
    return y


def tb_gemm(packing, packed, scales, xr, y=None, stream=None):
    """Y[M][N] = X'[M][K] (fp16) times the packed ternary weights, fp32 out."""
    _check(xr, "xr", (torch.float16,))
    _rank2(xr, "xr")
    m, k = xr.shape
    n = _weights(packing, packed, scales, k)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xr.device)
    _check(y, "y", (torch.float32,))
    _shape(y, "y", (m, n))
    _call("tb_gemm", _packing(packing), _ptr(packed), _ptr(scales), _ptr(xr), _ptr(y), m, n, k,
          _stream(stream))
    return y


def tb_ternarize(w, sign_bits=None, trits=None, scales=None, bad_count=None, stream=None):
    """fp32 weights W[N][K] -> (int8 trits [N][K], fp16 scales [N][K/128]) of W R_K^T
    (sign_bits=None: W is already in the rotated basis, the search alone)."""
    _check(w, "w", (torch.float32,))
    _rank2(w, "w")
    n, k = w.shape
    if k % 1024:
        raise ValueError(f"K = {k} is not a multiple of 1024")
    if sign_bits is not None:
        _signs(sign_bits, k)
    if trits is None:
        trits = torch.empty((n, k), dtype=torch.int8, device=w.device)
    if scales is None:
        scales = torch.empty((n, k // 128), dtype=torch.float16, device=w.device)
    _check(trits, "trits", (torch.int8,))
    _shape(trits, "trits", (n, k))
    _check(scales, "scales", (torch.float16,))
    _shape(scales, "scales", (n, k // 128))
    _count(bad_count)
    _call("tb_ternarize", _ptr(w), n, k, _ptr(sign_bits), _ptr(trits), _ptr(scales), _ptr(bad_count),
          _stream(stream))
    return trits, scales


def tb_stream_read(src, sink, nbytes=None, stream=None):
    """Read the first nbytes (default: all) of a device tensor once; the measured HBM ceiling."""
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _check(sink, "sink", (torch.int32,))
    total = src.numel() * src.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if not 0 <= nbytes <= total:
        raise ValueError(f"nbytes = {nbytes} outside 0..{total}")
    _call("tb_stream_read", _ptr(src), nbytes, _ptr(sink), sink.numel(), _stream(stream))


def tb_decode_chain(packing, linears, x0, sign_bits, sync, ys=None, spin_limit=0, stream=None):
    """Dependent batch-1 linears in one launch: linears = [(packed, scales), ...]; linear i > 0 reads
    the first K outputs of linear i - 1.  sync: int32 device tensor of at least len(linears) + 2
    words, zero before the first call.  Returns the outputs [y_0, ...] (fp32 [N_i])."""
    _check(x0, "x0", tuple(_ACT_DT))
    k = x0.numel()
    if x0.dim() not in (1, 2) or (x0.dim() == 2 and x0.shape[0] != 1):
        raise ValueError(f"x0 must be one activation row, got shape {tuple(x0.shape)}")
    _signs(sign_bits, k)
    _check(sync, "sync", (torch.int32,))
    if not 1 <= len(linears) <= TB_CHAIN_MAX:
        raise ValueError(f"1..{TB_CHAIN_MAX} linears, got {len(linears)}")
    arr = (ChainLinear * len(linears))()
    outs = []
    for i, (packed, scales) in enumerate(linears):
        n = _weights(packing, packed, scales, k)
        y = ys[i] if ys is not None else torch.empty(n, dtype=torch.float32, device=x0.device)
        _check(y, "y", (torch.float32,))
        _shape(y, "y", (n,))
        arr[i] = ChainLinear(packed.data_ptr(), scales.data_ptr(), y.data_ptr(), n)
        outs.append(y)
    _call("tb_decode_chain", _packing(packing), ctypes.cast(arr, ctypes.c_void_p), len(linears), _ptr(x0),
          _ACT_DT[x0.dtype], _ptr(sign_bits), k, _ptr(sync), sync.numel(), int(spin_limit), _stream(stream))
    return outs
