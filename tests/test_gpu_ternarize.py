"""The HIP ternariser (tb_ternarize) against the oracle's, through the C ABI.

Trits and fp16 scales are compared bit for bit: both sides rotate and search
in fp64, so the integer outcome can differ only at exact fp64 ties, which
these seeded inputs do not contain.  Expected values come only from the
oracle; inputs come from the seeded generator or are written out here.
"""
import numpy as np
import pytest
import torch

import fwht_rotation_sqrt_amd as tb
import oracle
import synth
from gpu_util import TOL, dev, host, note, signs_dev

pytestmark = pytest.mark.gpu


def _gpu(w32, sign_bits):
    w = dev(np.asarray(w32, dtype=np.float32))
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    sb = signs_dev(sign_bits) if sign_bits is not None else None
    t, s = tb.tb_ternarize(w, sb, bad_count=bad)
    return host(t), host(s).view(np.uint16), int(host(bad)[0])


def _assert_same(got, want):
    t, s, bad = got
    tr, sr, _, badr = want
    mism = np.argwhere(t != tr)
    assert len(mism) == 0, f"{len(mism)} trits differ, first at {mism[:4].tolist()}"
    ms = np.argwhere(s != sr)
    assert len(ms) == 0, f"{len(ms)} scales differ, first at {ms[:4].tolist()}: {s[tuple(ms[0])]:#x} vs {sr[tuple(ms[0])]:#x}"
    assert bad == badr


def _hand_groups():
    g = np.random.default_rng(31)
    signs = np.where(g.integers(0, 2, 128) == 1, -1.0, 1.0)
    groups = []
    groups.append(0.5 * signs)                                   # equal magnitudes
    w = np.full(128, 0.01)
    w[::8] = 1.0
    groups.append(w * signs)                                     # 16 large among 112 small
    groups.append(np.zeros(128))                                 # all zero
    w = np.full(128, 0.5)
    w[7] = np.nan
    groups.append(w)                                             # non-finite
    w = np.zeros(128)
    w[3] = 1e6
    groups.append(w)                                             # every candidate's scale overflows
    groups.append(np.full(128, 1e6) * signs)                     # only "keep nothing" is finite
    groups.append(np.full(128, 65504.0) * signs)                 # largest finite fp16 scale
    # mean kept magnitude 1 + 2^-11 + 2^-24: one rounding gives 1 + 2^-10 (via fp32: 1)
    w = np.where(np.arange(128) < 64, 1 + 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -23)
    groups.append(w * signs)
    w = np.where(np.arange(128) < 64, 2.0 ** -25, 2.0 ** -25 * (1 + 2.0 ** -15))
    groups.append(w * signs)                                     # fp16 subnormal scale, just above a tie
    k = np.full(128, 32)
    d = g.integers(-31, 32, size=64)
    k[:64] += d
    k[64:] -= d
    groups.append(k / 64 * signs)                                # every threshold equals a magnitude
    groups.append(g.standard_normal(128))
    groups.append(g.laplace(size=128) * 1e-3)
    groups.append(g.standard_t(3, size=128))
    sparse = np.zeros(128)
    sparse[g.choice(128, 5, replace=False)] = g.standard_normal(5)
    groups.append(sparse)
    groups.append(np.abs(g.standard_normal(128)))
    groups.append(g.standard_normal(128) * 2.0 ** 12)
    return np.concatenate(groups).reshape(1, 16 * 128).astype(np.float32)


def test_ternarize_hand_groups_search_only():
    note("ternarize hand groups, no rotation")
    w = _hand_groups()
    want = oracle.ternarize(w.astype(np.float64))
    assert want[3] == 2                                          # the NaN group and the overflowing one
    _assert_same(_gpu(w, None), want)


@pytest.mark.parametrize("n,k,std,outliers", [
    (1, 1024, 0.02, False), (3, 2048, 0.02, True), (17, 5120, 0.02, True), (64, 17408, 0.02, False),
    (5, 5120, 1e-6, False), (5, 5120, 1e3, True), (130, 1024, 1.0, True)])
def test_ternarize_rotated_parity(n, k, std, outliers):
    note(f"ternarize rotated n={n} k={k} std={std} outliers={outliers}")
    oc = synth.outlier_channels(synth.rng(300, synth.T_OUTLIERS, n % 251, k // 1024), k, 0.01) \
        if outliers else None
    w = synth.fp_weights(synth.rng(300, synth.T_FP_WEIGHTS, n % 251, k // 1024), n, k, std, oc)
    sb = synth.sign_bits(synth.rng(300, synth.T_SIGNS, 0, k // 1024), k)
    want = oracle.quantize_weights(w.astype(np.float64), sb)
    assert want[3] == 0
    _assert_same(_gpu(w, sb), want)


def test_ternarize_full_size_sampled_rows():
    n, k = synth.FFN, synth.HIDDEN
    note(f"ternarize full size {n}x{k}")
    oc = synth.outlier_channels(synth.rng(301, synth.T_OUTLIERS), k)
    w = synth.fp_weights(synth.rng(301, synth.T_FP_WEIGHTS), n, k, 0.02, oc)
    sb = synth.sign_bits(synth.rng(301, synth.T_SIGNS), k)
    t, s, bad = _gpu(w, sb)
    assert bad == 0
    rows = np.unique(np.concatenate([[0, 1, n - 1], synth.rng(301, 9).integers(0, n, 13)]))
    tr, sr, _, badr = oracle.quantize_weights(w[rows].astype(np.float64), sb)
    assert badr == 0
    assert (t[rows] == tr).all() and (s[rows] == sr).all()
    # every group holds some non-zero trit and a positive normal scale at this spread
    sv = s.view(np.float16).astype(np.float64)
    assert (sv > 6.1e-5).all() and np.isfinite(sv).all()


def test_ternarize_bad_blocks_and_count_accumulates():
    n, k = 4, 3072
    note(f"ternarize bad blocks n={n} k={k}")
    w = synth.fp_weights(synth.rng(302, synth.T_FP_WEIGHTS), n, k)
    w[1, 1500] = np.inf      # row 1, block 1: the rotation spreads it over the block's 8 groups
    w[3, 10] = np.nan        # row 3, block 0
    sb = synth.sign_bits(synth.rng(302, synth.T_SIGNS), k)
    want = oracle.quantize_weights(w.astype(np.float64), sb)
    assert want[3] == 16
    wd = dev(w)
    sbd = signs_dev(sb)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    t, s = tb.tb_ternarize(wd, sbd, bad_count=bad)
    _assert_same((host(t), host(s).view(np.uint16), int(host(bad)[0])), want)
    tb.tb_ternarize(wd, sbd, trits=t, scales=s, bad_count=bad)
    assert int(host(bad)[0]) == 32                               # added to, never reset
    assert (host(t)[1, 1024:2048] == 0).all() and (host(t)[3, :1024] == 0).all()


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_quantize_pack_linear_tracks_fp_product(packing):
    """fp weights -> tb_ternarize -> pack -> tb_linear: the product matches the oracle's
    product of the same quantised weights to TOL, and tracks W x at the quantiser's error."""
    n, k, b = 512, 5120, 4
    note(f"quantize + pack + linear {packing} n={n} k={k} b={b}")
    oc = synth.outlier_channels(synth.rng(303, synth.T_OUTLIERS), k, 0.01)
    w = synth.fp_weights(synth.rng(303, synth.T_FP_WEIGHTS), n, k, 0.02, oc)
    sb = synth.sign_bits(synth.rng(303, synth.T_SIGNS), k)
    x = synth.activations(synth.rng(303, synth.T_X), b, k, dtype="f32")
    t, s = tb.tb_ternarize(dev(w), signs_dev(sb))
    packed = tb.tb_pack_2bit(t) if packing == "2bit" else tb.tb_pack_base3(t)
    y = host(tb.tb_linear(packing, packed, s, dev(x), signs_dev(sb)))
    tr, sr, _, _ = oracle.quantize_weights(w.astype(np.float64), sb)
    pr, _ = oracle.pack_2bit(tr) if packing == "2bit" else oracle.pack_base3(tr)
    xr = oracle.rotate(x.astype(np.float64), sb)
    assert oracle.rel_err(y, oracle.gemv(packing, pr, sr, xr, k)) < TOL
    e = oracle.normwise_err(y, x.astype(np.float64) @ w.astype(np.float64).T)
    note(f"normwise error of W_hat (R x) against W x: {e:.4f}")
    assert 0.38 < e < 0.46
