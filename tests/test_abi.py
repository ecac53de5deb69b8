"""The C-ABI library loads and validates its arguments on the host (no GPU needed).

Every call here fails validation (or is an empty call), so no device work is
enqueued; pointers are plain integers that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

import fwht_rotation_sqrt_amd as tb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tb.h")

OK, NULL, SHAPE, ALIGN, DTYPE, UNSUP = 0, 1, 2, 3, 4, 5
P = 0x10000          # a 16-byte aligned fake address, never dereferenced
MIS = 0x10004        # a misaligned one


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int64_t|int|const char\*)\s+(tb_\w+)\s*\(", text, re.M)))


def test_header_declares_binding_exports():
    assert declared() == sorted(tb.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = tb.library()
    for name in declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", tb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (tb_\w+)", out))
    assert set(declared()) <= exported


def test_packed_row_bytes():
    lib = tb.library()
    assert lib.tb_packed_row_bytes(0, 5120) == 1280
    assert lib.tb_packed_row_bytes(1, 5120) == 1040
    assert lib.tb_packed_row_bytes(1, 17408) == 3536
    assert lib.tb_packed_row_bytes(0, 100) == -1
    assert lib.tb_packed_row_bytes(1, -128) == -1
    assert lib.tb_packed_row_bytes(7, 128) == -1


def test_pack_validation():
    lib = tb.library()
    for fn in (lib.tb_pack_2bit, lib.tb_pack_base3):
        assert fn(P, 4, 100, P, None, None) == SHAPE
        assert fn(P, -1, 128, P, None, None) == SHAPE
        assert fn(P, 4, 0, P, None, None) == SHAPE
        assert fn(None, 4, 128, P, None, None) == NULL
        assert fn(P, 4, 128, None, None, None) == NULL
        assert fn(P, 4, 128, MIS, None, None) == ALIGN
        assert fn(None, 0, 128, None, None, None) == OK          # empty call
    assert lib.tb_unpack(2, P, 4, 128, P, None, None) == UNSUP
    assert lib.tb_unpack(1, P, 4, 130, P, None, None) == SHAPE
    assert lib.tb_unpack(0, MIS, 4, 128, P, None, None) == ALIGN


def test_rotate_validation():
    lib = tb.library()
    f = lib.tb_fwht_rotate
    assert f(P, 0, P, 0, 2, 1000, P, None) == SHAPE
    assert f(P, 0, P, 0, 2, 128, P, None) == SHAPE
    assert f(P, 0, P, 0, -1, 1024, P, None) == SHAPE
    assert f(P, 5, P, 0, 2, 1024, P, None) == DTYPE
    assert f(P, 0, P, 2, 2, 1024, P, None) == DTYPE        # bf16 output not offered
    assert f(P, 2, P, 0, 2, 1024, P, None) == DTYPE        # in place needs equal dtypes
    assert f(None, 0, P, 0, 2, 1024, P, None) == NULL
    assert f(P, 0, P, 0, 2, 1024, None, None) == NULL
    assert f(P, 0, MIS, 0, 2, 1024, P, None) == ALIGN
    assert f(None, 0, None, 0, 0, 1024, None, None) == OK


def test_gemv_validation():
    lib = tb.library()
    g = lib.tb_gemv
    assert g(3, P, P, P, 0, P, 1, 8, 128, None) == UNSUP
    assert g(0, P, P, P, 0, P, 0, 8, 128, None) == SHAPE
    assert g(0, P, P, P, 0, P, tb.TB_GEMV_MAX_BATCH + 1, 8, 128, None) == SHAPE
    assert g(0, P, P, P, 0, P, 1, 8, 192, None) == SHAPE
    assert g(0, P, P, P, 0, P, 1, -8, 128, None) == SHAPE
    # 32 rows of K = 2^26 fp32 activations are 2^33 bytes: past the 32-bit offsets
    assert g(0, P, P, P, 0, P, 32, 8, 1 << 26, None) == SHAPE
    assert g(0, P, P, P, 2, P, 1, 8, 128, None) == DTYPE
    assert g(1, None, P, P, 0, P, 1, 8, 128, None) == NULL
    assert g(1, P, None, P, 0, P, 1, 8, 128, None) == NULL
    assert g(1, P, P, P, 0, None, 1, 8, 128, None) == NULL
    assert g(1, P, MIS, P, 0, P, 1, 8, 128, None) == ALIGN
    assert g(1, P, P, P, 0, P, 1, 0, 128, None) == OK
    assert g(1, P, P, P, 0, P, 1, 1 << 20, 1 << 12, None) == SHAPE   # > 2^31 weights


def test_linear_validation():
    lib = tb.library()
    g = lib.tb_linear
    # (packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, stream)
    assert g(3, P, P, P, 2, P, P, 1, 8, 1024, None) == UNSUP
    assert g(1, P, P, P, 2, P, P, 0, 8, 1024, None) == SHAPE
    assert g(1, P, P, P, 2, P, P, tb.TB_GEMV_MAX_BATCH + 1, 8, 1024, None) == SHAPE
    assert g(1, P, P, P, 2, P, P, 1, 8, 1152, None) == SHAPE      # K % 1024 != 0
    assert g(1, P, P, P, 2, P, P, 1, -8, 1024, None) == SHAPE
    assert g(1, P, P, P, 3, P, P, 1, 8, 1024, None) == DTYPE
    assert g(1, P, P, P, 2, None, P, 1, 8, 1024, None) == NULL    # sign bits
    assert g(1, None, P, P, 2, P, P, 1, 8, 1024, None) == NULL
    assert g(1, P, P, None, 2, P, P, 1, 8, 1024, None) == NULL
    assert g(1, P, P, P, 2, P, None, 1, 8, 1024, None) == NULL
    assert g(1, P, P, P, 2, MIS, P, 1, 8, 1024, None) == ALIGN
    assert g(0, P, P, MIS, 0, P, P, 1, 8, 1024, None) == ALIGN
    assert g(0, P, P, P, 1, P, P, 1, 0, 1024, None) == OK         # empty
    assert g(0, P, P, P, 0, P, P, 1, 1 << 20, 1 << 12, None) == SHAPE


def test_gemm_validation():
    lib = tb.library()
    g = lib.tb_gemm
    assert g(2, P, P, P, P, 4, 8, 128, None) == UNSUP
    assert g(1, P, P, P, P, 4, 8, 100, None) == SHAPE
    assert g(0, P, P, P, P, 4, 8, 100, None) == SHAPE
    assert g(0, P, P, P, P, -4, 8, 128, None) == SHAPE
    assert g(0, None, P, P, P, 4, 8, 128, None) == NULL
    assert g(0, P, P, MIS, P, 4, 8, 128, None) == ALIGN
    assert g(0, P, P, P, P, 0, 8, 128, None) == OK


def test_status_strings():
    lib = tb.library()
    for st in range(7):
        assert lib.tb_status_string(st)
    assert lib.tb_status_string(99) == b"unknown status"
    assert lib.tb_last_hip_error() == b""


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tb, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(tb, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        tb.library()
