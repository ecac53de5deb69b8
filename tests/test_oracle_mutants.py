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


def _rel_err_variant(mean=False, global_rms=False, cand_den=False, no_floor=False):
    def fn(orig, y, yref):
        y = np.asarray(y, dtype=np.float64)
        yref = np.asarray(yref, dtype=np.float64)
        yr = yref.reshape(-1, yref.shape[-1])
        yc = y.reshape(yr.shape)
        if not yr.size:
            return 0.0
        if global_rms:
            rms = np.sqrt(np.mean(yr * yr))
        else:
            rms = np.sqrt(np.mean(yr * yr, axis=1, keepdims=True))
        mag = np.abs(yc) if cand_den else np.abs(yr)
        den = mag if no_floor else np.maximum(mag, rms)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.abs(yc - yr) / np.where(den == 0, 1.0, den)
        return float(np.mean(ratio) if mean else np.max(ratio))
    return fn


def _normwise_per_row_max(orig, y, yref):
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    yref = np.atleast_2d(np.asarray(yref, dtype=np.float64))
    d = np.linalg.norm(yref, axis=-1)
    num = np.linalg.norm(y - yref, axis=-1)
    return float(np.max(np.where(d > 0, num / np.where(d > 0, d, 1), num)))


def _normwise_no_division(orig, y, yref):
    return float(np.linalg.norm(np.asarray(y, float) - np.asarray(yref, float)))


def _ternarize_variant(strict=False, mean_all=False, grid_from_zero=False, kept_error_only=False,
                       sign_flip=False, unrounded_error=False, last_on_ties=False):
    """The oracle's threshold search with one planted slip."""
    def fn(orig, wr):
        wr = np.asarray(wr, dtype=np.float64)
        n, k = wr.shape
        g = wr.reshape(-1, 128)
        mag = np.abs(g)
        finite = np.all(np.isfinite(g), axis=1)
        a = np.sum(np.where(finite[:, None], mag, 0.0), axis=1) / 128
        best = np.full(len(g), np.inf)
        bj = np.zeros(len(g), dtype=np.int64)
        bs = np.zeros(len(g), dtype=np.uint16)
        with np.errstate(over="ignore", invalid="ignore"):
            for j in range(64):
                c = j / 32 if grid_from_zero else (j + 1) / 32
                keep = mag > (c * a)[:, None] if strict else mag >= (c * a)[:, None]
                nnz = keep.sum(1)
                if mean_all:
                    s = a.copy()
                else:
                    s = np.divide(np.where(keep, mag, 0).sum(1), nnz, out=np.zeros(len(g)), where=nnz > 0)
                sb = o.f64_to_f16_bits(s)
                s16 = s if unrounded_error else sb.view(np.float16).astype(np.float64)
                kept = np.where(keep, (mag - s16[:, None]) ** 2, 0.0)
                err = (kept if kept_error_only else kept + np.where(keep, 0.0, mag * mag)).sum(1)
                better = (err <= best) if last_on_ties else (err < best)
                better |= j == 0
                best = np.where(better, err, best)
                bj = np.where(better, j, bj)
                bs = np.where(better, sb, bs)
            c = bj / 32 if grid_from_zero else (bj + 1) / 32
            keep = mag > (c * a)[:, None] if strict else mag >= (c * a)[:, None]
            t = np.where(keep, np.sign(g), 0.0).astype(np.int8)
            if sign_flip:
                t = -t
            bad = ~finite | ~np.isfinite(bs.view(np.float16))
            zero = (a == 0) | bad
            t[zero] = 0
            bs = np.where(zero, 0, bs).astype(np.uint16)
            bj = np.where(zero, -1, bj)
        return t.reshape(n, k), bs.reshape(n, k // 128), bj.reshape(n, k // 128), int(bad.sum())
    return fn


def _rotate_weights_untransposed(orig, w, sb):
    """W R_K instead of W R_K^T: each row times H S / 32 as a row vector."""
    w = np.asarray(w, dtype=float)
    k = w.shape[1]
    plus = np.zeros(k // 32, dtype=np.uint32)
    return o.rotate(w, plus) * o.sign_vector(sb, k)


MUTANTS = {
    "ternarize_strict_threshold": lambda mp: mp.setattr(
        o, *_wrap("ternarize", _ternarize_variant(strict=True))),
    "ternarize_scale_mean_of_all": lambda mp: mp.setattr(
        o, *_wrap("ternarize", _ternarize_variant(mean_all=True))),
    "ternarize_grid_from_zero": lambda mp: mp.setattr(
        o, *_wrap("ternarize", _ternarize_variant(grid_from_zero=True))),
    "ternarize_error_kept_only": lambda mp: mp.setattr(
        o, *_wrap("ternarize", _ternarize_variant(kept_error_only=True))),
    "ternarize_sign_flipped": lambda mp: mp.setattr(
        o, *_wrap("ternarize", _ternarize_variant(sign_flip=True))),
    "ternarize_last_on_ties": lambda mp: mp.setattr(
        o, *_wrap("ternarize", _ternarize_variant(last_on_ties=True))),
    "ternarize_unrounded_error": lambda mp: mp.setattr(
        o, *_wrap("ternarize", _ternarize_variant(unrounded_error=True))),
    "f16_via_f32": lambda mp: mp.setattr(
        o, *_wrap("f64_to_f16_bits", lambda orig, v: np.asarray(v, dtype=np.float64)
                  .astype(np.float32).astype(np.float16).view(np.uint16))),
    "rotate_weights_untransposed": lambda mp: mp.setattr(
        o, *_wrap("rotate_weights", _rotate_weights_untransposed)),
    "quantize_skips_rotation": lambda mp: mp.setattr(
        o, *_wrap("quantize_weights", lambda orig, w, sb: o.ternarize(w))),

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
    "rel_err_mean_for_max": lambda mp: mp.setattr(
        o, *_wrap("rel_err", _rel_err_variant(mean=True))),
    "rel_err_global_rms": lambda mp: mp.setattr(
        o, *_wrap("rel_err", _rel_err_variant(global_rms=True))),
    "rel_err_candidate_denominator": lambda mp: mp.setattr(
        o, *_wrap("rel_err", _rel_err_variant(cand_den=True))),
    "rel_err_floor_dropped": lambda mp: mp.setattr(
        o, *_wrap("rel_err", _rel_err_variant(no_floor=True))),
    "normwise_per_row": lambda mp: mp.setattr(o, *_wrap("normwise_err", _normwise_per_row_max)),
    "normwise_not_divided": lambda mp: mp.setattr(o, *_wrap("normwise_err", _normwise_no_division)),
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
