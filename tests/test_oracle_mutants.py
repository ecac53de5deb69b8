"""Planted mistakes in the oracle are caught by at least one pin.

Each mutant is a plausible slip (a reversed digit order, a dropped scale, a
wrong normalisation, a transposed operand...).  The mutant is applied to the
oracle module on the CPU only, for the duration of one test.
"""
import numpy as np
import pytest

import oracle.ternary as o
from conftest import read_golden
from oracle_pins import ALL_PINS


def _wrap(name, fn):
    orig = getattr(o, name)
    return name, (lambda *a, **kw: fn(orig, *a, **kw))


def _h_bitrev(n):
    h = ORIG_HADAMARD(n)
    bits = max(n.bit_length() - 1, 1)
    rev = [int(format(i, f"0{bits}b")[::-1], 2) for i in range(n)] if n > 1 else [0]
    return h[rev]


ORIG_HADAMARD = o.hadamard


def _pack2_msb_first(orig, trits):
    t, bad = o._check_trits(trits)
    n, k = t.shape
    c = (t + 1).reshape(n, k // 4, 4)
    return ((c[..., 3]) | (c[..., 2] << 2) | (c[..., 1] << 4) | (c[..., 0] << 6)).astype(np.uint8), bad


def _rotate_sign_after(orig, x, sb):
    x = np.asarray(x, dtype=float)
    k = x.shape[1]
    plus = np.zeros(k // 32, dtype=np.uint32)
    return orig(x, plus) * o.sign_vector(sb, k)


def _sign_vector_msb(orig, sb, k):
    w = np.asarray(sb, dtype=np.uint64)
    ch = np.arange(k)
    bit = (w[ch // 32] >> (31 - ch % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(bit == 1, -1.0, 1.0)


def _dequant_group64(orig, packing, packed, s, k):
    t, _ = o.unpack_2bit(packed, k) if packing == "2bit" else o.unpack_base3(packed, k)
    sv = np.asarray(s, dtype=np.uint16).view(np.float16).astype(float)
    idx = np.minimum(np.arange(k) // 64, sv.shape[1] - 1)
    return t * sv[:, idx]


def _dequant_no_scale(orig, packing, packed, s, k):
    t, _ = o.unpack_2bit(packed, k) if packing == "2bit" else o.unpack_base3(packed, k)
    return t.astype(float)


def _gemv_transposed(orig, packing, packed, s, xr, k):
    w = o.dequantize(packing, packed, s, k)
    return (np.asarray(xr, float) @ w.T)[:, ::-1]


def _pack3_pad_first(orig, trits):
    t, bad = o._check_trits(trits)
    n, k = t.shape
    g = t.reshape(n, k // 128, 128)
    g = np.concatenate([np.zeros((n, k // 128, 2), dtype=np.int64), g], axis=2)
    d = (g + 1).reshape(n, k // 128, 26, 5)
    return (d * o.POW3).sum(-1).reshape(n, -1).astype(np.uint8), bad


MUTANTS = {
    "base3_msd_first": lambda mp: mp.setattr(o, "POW3", o.POW3[::-1].copy()),
    "base3_pad_first": lambda mp: mp.setattr(o, *_wrap("pack_base3", _pack3_pad_first)),
    "2bit_msb_first": lambda mp: mp.setattr(o, *_wrap("pack_2bit", _pack2_msb_first)),
    "2bit_code_negated": lambda mp: mp.setattr(
        o, *_wrap("pack_2bit", lambda orig, t: orig(-np.asarray(t)))),
    "hadamard_bit_reversed_rows": lambda mp: mp.setattr(o, "hadamard", _h_bitrev),
    "rotate_scale_1_over_n": lambda mp: mp.setattr(
        o, *_wrap("rotate", lambda orig, x, sb: orig(x, sb) / 32)),
    "rotate_sign_after_h": lambda mp: mp.setattr(o, *_wrap("rotate", _rotate_sign_after)),
    "sign_bits_msb_first": lambda mp: mp.setattr(o, *_wrap("sign_vector", _sign_vector_msb)),
    "scale_group_64": lambda mp: mp.setattr(o, *_wrap("dequantize", _dequant_group64)),
    "scale_dropped": lambda mp: mp.setattr(o, *_wrap("dequantize", _dequant_no_scale)),
    "gemv_outputs_reversed": lambda mp: mp.setattr(o, *_wrap("gemv", _gemv_transposed)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(o, read_golden)
        except Exception:  # an assertion, or a shape error the mistake causes
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
