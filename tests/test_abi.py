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
    assert f(P, 0, P + 4096, 0, 2, 1024, P, None) == SHAPE  # rows overlap without being in place
    assert f(P + 4096, 2, P + 2048, 1, 2, 1024, P, None) == SHAPE
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


def test_linear_workspace_bytes():
    lib = tb.library()
    f = lib.tb_linear_workspace_bytes
    # (packing, B, N, K): the fused one-launch kernel below the measured crossover, x' in fp32 from
    # it on (K >= 8192: batch 2; else batch 5 base-3, 6 2-bit; never past the batched product's)
    assert f(0, 1, 17408, 5120) == 0 and f(1, 1, 17408, 5120) == 0
    assert f(0, 5, 17408, 5120) == 0 and f(0, 6, 17408, 5120) == 4 * 6 * 5120
    assert f(0, 9, 17408, 5120) == 4 * 9 * 5120
    assert f(1, 4, 17408, 5120) == 0 and f(1, 5, 17408, 5120) == 4 * 5 * 5120
    assert f(0, 5, 5120, 5120) == 0 and f(0, 6, 5120, 5120) == 4 * 6 * 5120
    assert f(1, 4, 5120, 5120) == 0 and f(1, 5, 5120, 5120) == 4 * 5 * 5120
    assert f(0, 1, 5120, 17408) == 0 and f(0, 2, 5120, 17408) == 4 * 2 * 17408
    assert f(1, 2, 5120, 17408) == 4 * 2 * 17408 and f(1, 2, 300, 8192) == 4 * 2 * 8192
    assert f(1, 4, 300, 7168) == 0 and f(1, 5, 300, 7168) == 4 * 5 * 7168
    # base-3 batch 1 with K past five 1024-blocks: partial sums of ceil(K / 5120) parts of K
    assert f(1, 1, 5120, 17408) == 4 * 4 * 5120 and f(1, 1, 5120, 6144) == 4 * 2 * 5120
    assert f(1, 1, 777, 11264) == 4 * 3 * 777 and f(1, 1, 40000, 17408) == 4 * 4 * 40000
    assert f(1, 1, 5120, 5120) == 0
    # from the batched product's batch on, x' plus the partial sums of its parts of K where the rows
    # are too few for five-tile workgroups on every compute unit (5120 rows: four parts; 9000 rows:
    # two parts from batch 16; 17408 rows: whole rows)
    assert f(1, 32, 5120, 17408) == 4 * 32 * 17408 + 4 * 4 * 32 * 5120
    assert f(1, 8, 5120, 5120) == 4 * 8 * 5120 + 4 * 4 * 8 * 5120
    assert f(1, 8, 300, 17408) == 4 * 8 * 17408 + 4 * 8 * 8 * 300       # 8 parts (at most 8)
    assert f(1, 8, 300, 2048) == 4 * 8 * 2048                           # 16 groups: 2 parts below 16 rows
    assert f(1, 16, 300, 2048) == 4 * 16 * 2048 + 4 * 2 * 16 * 300
    assert f(0, 9, 9000, 5120) == 4 * 9 * 5120 and f(0, 16, 9000, 5120) == 4 * 16 * 5120 + 4 * 2 * 16 * 9000
    assert f(1, 32, 17408, 5120) == 4 * 32 * 5120
    assert f(1, 33, 8, 1024) == -1 and f(1, 0, 8, 1024) == -1 and f(1, 4, 8, 1152) == -1
    assert f(2, 4, 8, 1024) == -1 and f(1, 4, -1, 1024) == -1


def test_linear_ws_validation():
    lib = tb.library()
    g = lib.tb_linear_ws
    # (packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, workspace, workspace_bytes, stream)
    need = 4 * 16 * 1024
    assert g(3, P, P, P, 2, P, P, 16, 8, 1024, P, need, None) == UNSUP
    assert g(1, P, P, P, 2, P, P, 33, 8, 1024, P, need, None) == SHAPE
    assert g(1, P, P, P, 2, P, P, 16, 8, 1152, P, need, None) == SHAPE
    assert g(1, P, P, P, 2, P, P, 16, -8, 1024, P, need, None) == SHAPE
    assert g(1, P, P, P, 3, P, P, 16, 8, 1024, P, need, None) == DTYPE
    assert g(1, P, P, P, 2, P, P, 16, 8, 1024, P, need - 1, None) == 7   # TB_ERR_WORKSPACE
    assert g(1, P, P, P, 2, P, P, 16, 8, 1024, None, need, None) == NULL
    assert g(1, P, P, P, 2, None, P, 16, 8, 1024, P, need, None) == NULL
    assert g(1, P, P, P, 2, P, P, 16, 8, 1024, MIS, need, None) == ALIGN
    assert g(1, P, P, P, 2, P, P, 16, 8, 1024, P, need, None) == SHAPE   # x is the workspace
    Q = P + 0x100000
    # x [16][1024] bf16 is 32 KiB from P: a workspace starting inside it, or ending inside y
    assert g(1, P, P, P, 2, P, Q, 16, 8, 1024, P + 0x4000, need, None) == SHAPE
    assert g(1, P, P, P, 2, P, Q, 16, 8, 1024, Q - need + 16, need, None) == SHAPE
    # batch 1, base-3, K = 17408: the partial sums (4 x 4 x 8 bytes) may not overlap y either
    assert g(1, P, P, P, 2, P, Q, 1, 8, 17408, Q + 16, 4 * 4 * 8, None) == SHAPE
    assert g(1, P, P, P, 2, P, P, 16, 0, 1024, P + 0x100000, need, None) == OK   # empty
    # batches the fused kernel serves need no workspace and behave as tb_linear
    assert g(1, P, P, P, 3, P, P, 1, 8, 1024, None, 0, None) == DTYPE
    assert g(1, P, P, P, 2, P, P, 1, 0, 1024, None, 0, None) == OK


def test_linear_noalloc_validation():
    lib = tb.library()
    g = lib.tb_linear_noalloc
    # (packing, packed, scales, x, x_dtype, sign_bits, y, B, N, K, stream): errors before any device call
    assert g(3, P, P, P, 2, P, P, 16, 8, 1024, None) == UNSUP
    assert g(1, P, P, P, 2, P, P, 33, 8, 1024, None) == SHAPE
    assert g(1, P, P, P, 2, P, P, 32, 8, 1 << 16, None) == 8          # B K = 2^21 > the static 2^20 floats
    assert g(1, P, P, P, 3, P, P, 1, 8, 1024, None) == DTYPE          # batch the fused kernel serves
    assert g(1, P, P, P, 2, None, P, 1, 8, 1024, None) == NULL


def test_decode_chain_validation():
    lib = tb.library()
    g = lib.tb_decode_chain
    Lin = tb.ChainLinear

    def arr(*ns, p=P):
        a = (Lin * len(ns))()
        for i, n in enumerate(ns):
            a[i] = Lin(p, p, p, n)
        return a

    two = arr(2048, 512)
    # (packing, linears, count, x0, x_dtype, sign_bits, K, sync, sync_words, spin_limit, stream)
    assert g(3, two, 2, P, 2, P, 1024, P, 4, 0, None) == UNSUP
    assert g(1, two, 0, P, 2, P, 1024, P, 4, 0, None) == SHAPE
    assert g(1, two, tb.TB_CHAIN_MAX + 1, P, 2, P, 1024, P, 4, 0, None) == SHAPE
    assert g(1, two, 2, P, 2, P, 1000, P, 4, 0, None) == SHAPE              # K % 1024 != 0
    assert g(1, arr(512, 2048), 2, P, 2, P, 1024, P, 4, 0, None) == SHAPE   # an inner N below K
    assert g(1, arr(0), 1, P, 2, P, 1024, P, 3, 0, None) == SHAPE
    assert g(1, None, 2, P, 2, P, 1024, P, 4, 0, None) == NULL
    assert g(1, arr(2048, 512, p=0), 2, P, 2, P, 1024, P, 4, 0, None) == NULL
    assert g(1, arr(2048, 512, p=MIS), 2, P, 2, P, 1024, P, 4, 0, None) == ALIGN
    assert g(1, two, 2, P, 3, P, 1024, P, 4, 0, None) == DTYPE
    assert g(1, two, 2, None, 2, P, 1024, P, 4, 0, None) == NULL
    assert g(1, two, 2, P, 2, P, 1024, None, 4, 0, None) == NULL
    assert g(1, two, 2, P, 2, MIS, 1024, P, 4, 0, None) == ALIGN
    assert g(1, two, 2, P, 2, P, 1024, P, 3, 0, None) == 7                  # sync needs count + 2 words
    assert g(0, two, 2, P, 2, P, 1024, P, 4, 0, None) == UNSUP              # 2-bit codes
    assert g(1, arr(8192, 512), 2, P, 2, P, 6144, P, 4, 0, None) == UNSUP   # K > 5120


def test_ternarize_validation():
    lib = tb.library()
    g = lib.tb_ternarize
    # (w, N, K, sign_bits, trits, scales, bad_count, stream)
    assert g(P, 4, 1152, P, P, P, None, None) == SHAPE             # K % 1024 != 0
    assert g(P, -1, 1024, P, P, P, None, None) == SHAPE
    assert g(P, 4, 0, P, P, P, None, None) == SHAPE
    assert g(P, 1 << 20, 1 << 12, P, P, P, None, None) == SHAPE   # N K beyond 32-bit offsets
    assert g(None, 4, 1024, P, P, P, None, None) == NULL
    assert g(P, 4, 1024, P, None, P, None, None) == NULL
    assert g(P, 4, 1024, P, P, None, None, None) == NULL
    assert g(MIS, 4, 1024, P, P, P, None, None) == ALIGN
    assert g(P, 4, 1024, MIS, P, P, None, None) == ALIGN
    assert g(P, 4, 1024, P, P, MIS, None, None) == ALIGN
    assert g(None, 0, 1024, None, None, None, None, None) == OK   # empty call


def test_stream_read_validation():
    lib = tb.library()
    g = lib.tb_stream_read
    assert g(P, -1, P, 8192, None) == SHAPE
    assert g(P, 1 << 31, P, 8192, None) == SHAPE
    assert g(P, 1000, P, 8192, None) == SHAPE         # not a multiple of 16
    assert g(None, 1024, P, 8192, None) == NULL
    assert g(P, 1024, None, 8192, None) == NULL
    assert g(MIS, 1024, P, 8192, None) == ALIGN
    assert g(P, 1 << 30, P, 100, None) == 7          # the sink is too small for the grid
    assert g(None, 0, None, 0, None) == OK


def test_status_strings():
    lib = tb.library()
    for st in range(9):
        assert lib.tb_status_string(st) != b"unknown status"
    assert lib.tb_status_string(99) == b"unknown status"
    assert lib.tb_last_hip_error() == b""


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tb, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(tb, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        tb.library()
