"""The Python binding rejects mismatched tensor shapes before any launch.

The kernels size every read and write from the integer arguments, so a
packed array, scale array, sign mask or output of the wrong shape must be
refused on the host with ValueError.  Only small device tensors are
allocated; no kernel runs in these tests.
"""
import pytest
import torch

import fwht_rotation_sqrt_amd as tb

pytestmark = pytest.mark.gpu

D = "cuda"


def _w(packing, n, k, rb_delta=0, sc_delta=0):
    rb = tb.tb_packed_row_bytes(packing, k) + rb_delta
    packed = torch.zeros((n, rb), dtype=torch.uint8, device=D)
    scales = torch.zeros((n, k // 128 + sc_delta), dtype=torch.float16, device=D)
    return packed, scales


def test_gemv_shape_errors():
    n, k = 16, 1024
    xr = torch.zeros((1, k), dtype=torch.float32, device=D)
    # a base-3 array (26 bytes per group) passed as 2-bit (32 bytes per group)
    packed, scales = _w("base3", n, k)
    with pytest.raises(ValueError, match="packed"):
        tb.tb_gemv("2bit", packed, scales, xr)
    packed, scales = _w("2bit", n, k, sc_delta=-1)
    with pytest.raises(ValueError, match="scales"):
        tb.tb_gemv("2bit", packed, scales, xr)
    packed, scales = _w("2bit", n, k)
    with pytest.raises(ValueError, match="y"):
        tb.tb_gemv("2bit", packed, scales, xr, y=torch.zeros((1, n - 1), device=D))
    with pytest.raises(ValueError, match="packed"):
        tb.tb_gemv("2bit", packed[:, :-1].contiguous(), scales, xr)
    with pytest.raises(ValueError):
        tb.tb_gemv("2bit", packed, scales, torch.zeros((1, 1000), device=D))


def test_linear_shape_errors():
    n, k = 16, 2048
    x = torch.zeros((2, k), dtype=torch.bfloat16, device=D)
    signs = torch.zeros(k // 32, dtype=torch.int32, device=D)
    packed, scales = _w("base3", n, k)
    with pytest.raises(ValueError, match="sign_bits"):
        tb.tb_linear("base3", packed, scales, x, signs[:-1].contiguous())
    with pytest.raises(ValueError, match="packed"):
        tb.tb_linear("2bit", packed, scales, x, signs)
    with pytest.raises(ValueError, match="y"):
        tb.tb_linear("base3", packed, scales, x, signs, y=torch.zeros((1, n), device=D))
    packed, scales = _w("base3", n, k, sc_delta=1)
    with pytest.raises(ValueError, match="scales"):
        tb.tb_linear("base3", packed, scales, x, signs)


def test_gemm_shape_errors():
    n, k, m = 16, 1024, 130
    xr = torch.zeros((m, k), dtype=torch.float16, device=D)
    packed, scales = _w("2bit", n, k, rb_delta=-16)
    with pytest.raises(ValueError, match="packed"):
        tb.tb_gemm("2bit", packed, scales, xr)
    packed, scales = _w("2bit", n, k)
    with pytest.raises(ValueError, match="y"):
        tb.tb_gemm("2bit", packed, scales, xr, y=torch.zeros((m, n + 1), device=D))


def test_rotate_pack_unpack_shape_errors():
    k = 1024
    x = torch.zeros((3, k), dtype=torch.float32, device=D)
    signs = torch.zeros(k // 32, dtype=torch.int32, device=D)
    with pytest.raises(ValueError, match="sign_bits"):
        tb.tb_fwht_rotate(x, torch.zeros(k // 64, dtype=torch.int32, device=D))
    with pytest.raises(ValueError, match="out"):
        tb.tb_fwht_rotate(x, signs, out=torch.zeros((2, k), device=D))
    trits = torch.zeros((4, 256), dtype=torch.int8, device=D)
    with pytest.raises(ValueError, match="packed"):
        tb.tb_pack_base3(trits, packed=torch.zeros((4, 64), dtype=torch.uint8, device=D))
    with pytest.raises(ValueError, match="bad_count"):
        tb.tb_pack_2bit(trits, bad_count=torch.zeros(0, dtype=torch.int32, device=D))
    packed = torch.zeros((4, 52), dtype=torch.uint8, device=D)       # base-3, K = 256
    with pytest.raises(ValueError, match="packed"):
        tb.tb_unpack("2bit", packed, 256)
    with pytest.raises(ValueError, match="trits"):
        tb.tb_unpack("base3", packed, 256, trits=torch.zeros((4, 128), dtype=torch.int8, device=D))
