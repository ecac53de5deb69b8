"""Pins of the oracle to facts fixed outside it (helper module, not collected).

Each pin takes the oracle module ``o`` (``oracle.ternary``) and raises
AssertionError when the oracle disagrees with something the pages or the
mathematics fix: values printed on the pages, closed forms, invariants, an
independent construction, or brute force on tiny inputs.  The same pins run
against deliberately broken copies of the oracle in test_oracle_mutants.py,
which shows that a plausible mistake anywhere in it makes at least one pin fail.
"""
from __future__ import annotations

import itertools

import numpy as np

import synth


# ------------------------------------------------------------------ base-3 code

def pin_base3_page_example(o, read_golden):
    """The worked example of the learning-path page: [-1,0,1,-1,1] -> 183 and back."""
    keyed, _ = read_golden("base3_worked_example.txt")
    five = keyed["trits"]
    row = np.zeros((1, 128), dtype=np.int8)
    row[0, :5] = five
    packed, bad = o.pack_base3(row)
    assert bad == 0
    assert int(packed[0, 0]) == keyed["byte"][0]
    back, bad = o.unpack_base3(packed, 128)
    assert bad == 0 and back[0, :5].tolist() == five


def pin_base3_bijection(o, read_golden=None):
    """All 3**5 = 243 five-trit tuples get distinct bytes < 243 that decode back.

    The byte of a tuple is also its value as a base-3 numeral with the first
    trit least significant (Python's int(str, 3) reads most significant first).
    """
    tuples = list(itertools.product((-1, 0, 1), repeat=5))
    per_group = 25
    groups = -(-len(tuples) // per_group)
    row = np.zeros((1, groups * 128), dtype=np.int8)
    for i, tup in enumerate(tuples):
        g, j = divmod(i, per_group)
        row[0, g * 128 + 5 * j: g * 128 + 5 * j + 5] = tup
    packed, bad = o.pack_base3(row)
    assert bad == 0
    got = []
    for i, tup in enumerate(tuples):
        g, j = divmod(i, per_group)
        b = int(packed[0, g * 26 + j])
        numeral = "".join(str(t + 1) for t in reversed(tup))
        assert b == int(numeral, 3), (tup, b)
        got.append(b)
    assert sorted(got) == list(range(243))
    back, bad = o.unpack_base3(packed, row.shape[1])
    assert bad == 0 and np.array_equal(back, row)


def pin_base3_pad_and_size(o, read_golden=None):
    """26 bytes per 128-group; last byte = d0 + 3 d1 + 9 d2 + 108 lies in 108..134."""
    g = synth.rng(90, 0)
    t = synth.trits(g, 5, 1024)
    packed, bad = o.pack_base3(t)
    assert bad == 0 and packed.shape == (5, 26 * 8)
    last = packed.reshape(5, 8, 26)[..., 25].astype(int)
    assert last.min() >= 108 and last.max() <= 134
    tail = t.reshape(5, 8, 128)[..., 125:].astype(int) + 1
    assert np.array_equal(last, tail[..., 0] + 3 * tail[..., 1] + 9 * tail[..., 2] + 108)
    assert np.all(packed < 243)


def pin_base3_bad_counts(o, read_golden=None):
    t = np.zeros((1, 128), dtype=np.int8)
    t[0, 7] = 2
    t[0, 9] = -3
    packed, bad = o.pack_base3(t)
    assert bad == 2 and int(packed[0, 1]) == 121          # byte 1 holds trits 5..9, all 0
    p = packed.copy()
    p[0, 3] = 250                                          # not a base-3 code
    p[0, 25] = 27 * 0 + 81 * 1 + 13                        # pad digits (0, 1): bad pad
    back, bad = o.unpack_base3(p, 128)
    assert bad == 2
    assert back[0, 15:20].tolist() == [0] * 5


# ------------------------------------------------------------------ 2-bit code

def pin_2bit_base4_number(o, read_golden=None):
    """A packed row is the little-endian base-4 numeral sum_k (t_k + 1) 4**k."""
    t = synth.trits(synth.rng(91, 0), 3, 256)
    packed, bad = o.pack_2bit(t)
    assert bad == 0 and packed.shape == (3, 64)
    for r in range(3):
        value = sum(int(c + 1) * 4 ** k for k, c in enumerate(t[r]))
        assert int.from_bytes(packed[r].tobytes(), "little") == value
    # hand example: trits (-1, 0, 1, -1) -> codes (0, 1, 2, 0) -> 0b00_10_01_00 = 0x24
    row = np.zeros((1, 128), dtype=np.int8)
    row[0, :4] = (-1, 0, 1, -1)
    assert int(o.pack_2bit(row)[0][0, 0]) == 0x24


def pin_2bit_bijection(o, read_golden=None):
    """The 81 valid bytes are exactly the bytes with no 11 field, and decode back."""
    tuples = list(itertools.product((-1, 0, 1), repeat=4))
    row = np.zeros((1, 384), dtype=np.int8)
    for i, tup in enumerate(tuples):
        row[0, 4 * i: 4 * i + 4] = tup
    packed, bad = o.pack_2bit(row)
    assert bad == 0
    got = sorted(int(b) for b in packed[0, :81])
    valid = [b for b in range(256) if all(((b >> (2 * i)) & 3) != 3 for i in range(4))]
    assert got == valid
    back, bad = o.unpack_2bit(packed, 384)
    assert bad == 0 and np.array_equal(back, row)


def pin_2bit_bad_counts(o, read_golden=None):
    row = np.zeros((1, 128), dtype=np.int8)
    row[0, 0] = 5
    packed, bad = o.pack_2bit(row)
    assert bad == 1 and int(packed[0, 0]) == 0x55
    p = packed.copy()
    p[0, 1] = 0xFF                                          # four 11 codes
    back, bad = o.unpack_2bit(p, 128)
    assert bad == 4 and back[0, 4:8].tolist() == [0, 0, 0, 0]


def pin_bits_per_weight(o, read_golden=None):
    """bits = bytes * 8 / params: 2 + 1/8 for 2-bit, 26*8/128 + 1/8 = 1.75 for base-3."""
    for k in (1024, 5120, 17408):
        assert o.bits_per_weight("2bit", k) == 2.125
        assert o.bits_per_weight("base3", k) == 1.75
        assert o.bits_per_weight("base3", k, with_scales=False) == 1.625
    assert o.packed_row_bytes("base3", 5120) == 1040 and o.packed_row_bytes("2bit", 5120) == 1280
    assert o.packed_row_bytes("2bit", 1000) == -1


# ------------------------------------------------------------------ Hadamard / rotation

def sylvester(n):
    """Independent construction: H_1 = [1], H_2m = [[H, H], [H, -H]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def pin_hadamard_page_h4(o, read_golden):
    _, rows = read_golden("hadamard4.txt")
    assert np.array_equal(o.hadamard(4), np.array(rows, dtype=float))


def pin_hadamard_sylvester(o, read_golden=None):
    for n in (1, 2, 8, 64, 1024):
        h = o.hadamard(n)
        assert np.array_equal(h, sylvester(n))
        assert np.array_equal(h, h.T)
        assert np.array_equal(h @ h.T, n * np.eye(n))


def _signs(seed=92, k=1024):
    return synth.sign_bits(synth.rng(seed, synth.T_SIGNS), k)


def pin_rotation_orthogonal(o, read_golden=None):
    """R R^T = I and |Rx| = |x| (R is orthogonal)."""
    sb = _signs()
    rt = o.rotate(np.eye(1024), sb)           # row i = R e_i, i.e. R^T
    assert np.max(np.abs(rt @ rt.T - np.eye(1024))) < 1e-12
    x = synth.rng(92, 9).standard_normal((3, 2048))
    sb2 = _signs(k=2048)
    y = o.rotate(x, sb2)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def pin_rotation_closed_forms(o, read_golden=None):
    """R e_j = S_jj H[:, j] / 32 (entries exactly +-1/32); R (S 1) = 32 e_0."""
    sb = _signs()
    s = o.sign_vector(sb, 1024)
    bits = [(int(sb[j // 32]) >> (j % 32)) & 1 for j in range(1024)]
    assert np.array_equal(s, np.array([-1.0 if b else 1.0 for b in bits]))
    h = sylvester(1024)
    for j in (0, 1, 5, 511, 1023):
        e = np.zeros((1, 1024))
        e[0, j] = 1
        assert np.array_equal(o.rotate(e, sb)[0], s[j] * h[:, j] / 32)
    ones = o.rotate(s[None, :], sb)[0]
    want = np.zeros(1024)
    want[0] = 32
    assert np.array_equal(ones, want)
    # blocks are independent and share the sign diagonal
    sb3 = _signs(k=3072)
    x = np.zeros((1, 3072))
    x[0, 2048 + 3] = 1
    y = o.rotate(x, sb3)[0]
    assert np.all(y[:2048] == 0) and np.array_equal(y[2048:], s[3] * h[:, 3] / 32)


def _butterfly(v):
    """Fast Walsh-Hadamard transform by butterflies, divided by sqrt(n)  [P4 section 5.2]."""
    v = np.array(v, dtype=np.float64)
    n = v.shape[-1]
    span = 1
    idx = np.arange(n)
    while span < n:
        lo = idx[(idx & span) == 0]
        a, b = v[..., lo].copy(), v[..., lo + span].copy()
        v[..., lo], v[..., lo + span] = a + b, a - b
        span *= 2
    return v / np.sqrt(n)


def pin_rotation_butterfly(o, read_golden=None):
    """Explicit product == O(n log n) butterfly on S x, per block."""
    sb = _signs(k=2048)
    s = o.sign_vector(sb, 2048)
    x = synth.rng(93, 1).standard_normal((4, 2048))
    y = o.rotate(x, sb)
    z = _butterfly((x * s).reshape(4, 2, 1024)).reshape(4, 2048)
    assert np.max(np.abs(y - z)) < 1e-12


def pin_rotation_inverse(o, read_golden=None):
    """S H (R x) / 32 = x."""
    sb = _signs()
    s = o.sign_vector(sb, 1024)
    x = synth.rng(93, 2).standard_normal((2, 1024))
    back = (o.rotate(x, sb) @ sylvester(1024)) / 32 * s
    assert np.max(np.abs(back - x)) < 1e-12


# ------------------------------------------------------------------ products

def _brute_gemv(t, s_bits, xr):
    """Pure-Python loops from the trits themselves (no packing involved)."""
    s = synth.f16_bits_to_f64(s_bits)
    rows, k = xr.shape
    n = t.shape[0]
    y = [[0.0] * n for _ in range(rows)]
    for b in range(rows):
        for r in range(n):
            acc = 0.0
            for gi in range(k // 128):
                part = 0.0
                for kk in range(gi * 128, gi * 128 + 128):
                    part += int(t[r, kk]) * float(xr[b, kk])
                acc += float(s[r, gi]) * part
            y[b][r] = acc
    return np.array(y)


def pin_gemv_bruteforce(o, read_golden=None):
    for packing in ("2bit", "base3"):
        for n, k, rows in ((1, 1024, 1), (3, 1024, 2), (7, 2048, 1)):
            g = synth.rng(94, 0, n, k // 1024)
            t = synth.trits(g, n, k)
            s = synth.scales_f16(g, n, k)
            xr = g.standard_normal((rows, k))
            packed, _ = o.pack_2bit(t) if packing == "2bit" else o.pack_base3(t)
            y = o.gemv(packing, packed, s, xr, k)
            assert y.shape == (rows, n)
            ref = _brute_gemv(t, s, xr)
            assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def pin_gemv_associativity(o, read_golden=None):
    """W_hat (R_K x) == (W_hat R_K) x with R_K built column by column."""
    k, n = 2048, 5
    g = synth.rng(95, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    sb = _signs(k=k)
    x = g.standard_normal((2, k))
    for packing in ("2bit", "base3"):
        packed, _ = o.pack_2bit(t) if packing == "2bit" else o.pack_base3(t)
        y = o.gemv(packing, packed, s, o.rotate(x, sb), k)
        w = t.astype(float) * np.repeat(synth.f16_bits_to_f64(s), 128, axis=1)
        r_t = o.rotate(np.eye(k), sb)                  # R_K^T
        y2 = x @ (w @ r_t.T).T
        assert np.max(np.abs(y - y2)) < 1e-12


def pin_gemv_unit_inputs(o, read_golden=None):
    """x' = e_j gives y_n = s[n][j//128] t[n][j] exactly; x = R^T e_j end to end too."""
    k, n = 1024, 6
    g = synth.rng(96, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    sv = synth.f16_bits_to_f64(s)
    sb = _signs()
    sgn = o.sign_vector(sb, k)
    h = sylvester(k)
    for packing in ("2bit", "base3"):
        packed, _ = o.pack_2bit(t) if packing == "2bit" else o.pack_base3(t)
        for j in (0, 127, 128, 700, 1023):
            e = np.zeros((1, k))
            e[0, j] = 1
            want = np.array([sv[r, j // 128] * t[r, j] for r in range(n)])
            assert np.array_equal(o.gemv(packing, packed, s, e, k)[0], want)
            x = sgn * h[:, j] / 32                    # R^T e_j, so R x = e_j
            y = o.gemv(packing, packed, s, o.rotate(x[None, :], sb), k)[0]
            assert np.max(np.abs(y - want)) < 1e-15


def pin_gemv_zero_and_linearity(o, read_golden=None):
    k, n = 1024, 4
    g = synth.rng(97, 0)
    s = synth.scales_f16(g, n, k)
    x = g.standard_normal((1, k))
    zeros = np.zeros((n, k), dtype=np.int8)
    for packing in ("2bit", "base3"):
        packed, _ = o.pack_2bit(zeros) if packing == "2bit" else o.pack_base3(zeros)
        assert np.all(o.gemv(packing, packed, s, x, k) == 0)
    t = synth.trits(g, n, k)
    x2 = g.standard_normal((1, k))
    for packing in ("2bit", "base3"):
        packed, _ = o.pack_2bit(t) if packing == "2bit" else o.pack_base3(t)
        y1 = o.gemv(packing, packed, s, x, k)
        y2 = o.gemv(packing, packed, s, x2, k)
        y12 = o.gemv(packing, packed, s, 3 * x - 0.5 * x2, k)
        assert np.max(np.abs(y12 - (3 * y1 - 0.5 * y2))) < 1e-12
        s2 = (synth.f16_bits_to_f64(s) * 2).astype(np.float16).view(np.uint16)
        assert np.array_equal(o.gemv(packing, packed, s2, x, k), 2 * y1)


def pin_gemm_rows_are_gemv(o, read_golden=None):
    k, n, m = 1024, 9, 5
    g = synth.rng(98, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    x = g.standard_normal((m, k))
    packed, _ = o.pack_2bit(t)
    y = o.gemm("2bit", packed, s, x, k)
    assert y.shape == (m, n)
    for r in range(m):
        yr = o.gemv("2bit", packed, s, x[r:r + 1], k)[0]
        assert np.max(np.abs(y[r] - yr)) <= 1e-13 * np.max(np.abs(yr))


# ------------------------------------------------------------------ comparison metric
#
# Every product parity verdict goes through rel_err: e = max_i |y_i - yref_i| /
# max(|yref_i|, rms of yref's row), the reading of the "max relative error 2e-3"
# bound in which an output that cancels to near zero is measured against its
# row's rms.  The cases below are small enough to work out by hand.

def pin_rel_err_hand_cases(o, read_golden=None):
    # one row, floor active: rms([3, 4, 0]) = sqrt(25/3); the error sits on the 0
    e = o.rel_err(np.array([[3.0, 4.0, 0.01]]), np.array([[3.0, 4.0, 0.0]]))
    assert abs(e - 0.01 / np.sqrt(25 / 3)) < 1e-15
    # floor inactive: |yref| = 4 > rms, so the error is relative to 4
    e = o.rel_err(np.array([[3.0, 4.004, 0.0]]), np.array([[3.0, 4.0, 0.0]]))
    assert abs(e - 0.004 / 4) < 1e-15
    # the rms is per row: a small row is not floored by a large row's rms
    yref = np.array([[1000.0, -1000.0], [1.0, 1.0]])
    y = np.array([[1000.0, -1000.0], [1.002, 1.0]])
    assert abs(o.rel_err(y, yref) - 0.002) < 1e-12
    # maximum, not mean, over the elements
    yref = np.ones((1, 4))
    y = np.array([[1.002, 1.0, 1.0, 1.0]])
    assert abs(o.rel_err(y, yref) - 0.002) < 1e-12
    # the denominator is the reference's, not the candidate's
    y = np.array([[1.0, 1.0, 1.0, 11.0]])
    assert o.rel_err(y, yref) == 10.0
    # a reference exactly 0 next to a non-zero entry: the floor is rms = sqrt(2)
    e = o.rel_err(np.array([[1e-3, 2.0]]), np.array([[0.0, 2.0]]))
    assert abs(e - 1e-3 / np.sqrt(2)) < 1e-15
    # leading dimensions are rows: [2][1][3] is two rows of three
    yref = np.array([[[3.0, 4.0, 0.0]], [[300.0, 400.0, 0.0]]])
    y = yref.copy()
    y[1, 0, 2] = 1.0
    assert abs(o.rel_err(y, yref) - 1.0 / np.sqrt(250000 / 3)) < 1e-15
    # an all-zero reference row: the error is absolute
    assert o.rel_err(np.array([[0.5, 0.0]]), np.zeros((1, 2))) == 0.5
    assert o.rel_err(np.zeros((1, 2)), np.zeros((1, 2))) == 0.0
    # exact agreement and the empty call
    assert o.rel_err(yref, yref) == 0.0
    assert o.rel_err(np.zeros((0, 5)), np.zeros((0, 5))) == 0.0
    # non-finite outputs never pass a bound
    for bad in (np.nan, np.inf, -np.inf):
        y = np.ones((1, 4))
        y[0, 2] = bad
        e = o.rel_err(y, np.ones((1, 4)))
        assert not (e < 1e30)


def pin_normwise_err_hand_cases(o, read_golden=None):
    # |(3, 4.5) - (3, 4)| / |(3, 4)| = 0.5 / 5
    assert abs(o.normwise_err(np.array([3.0, 4.5]), np.array([3.0, 4.0])) - 0.1) < 1e-15
    # over the whole array, not row by row: |(0, 0, 0, 0.1)| / |(3, 4, 0.3, 0.4)|
    y = np.array([[3.0, 4.0], [0.3, 0.5]])
    yref = np.array([[3.0, 4.0], [0.3, 0.4]])
    assert abs(o.normwise_err(y, yref) - 0.1 / np.sqrt(25.25)) < 1e-14
    # a zero reference gives the norm of y itself
    assert o.normwise_err(np.array([3.0, 4.0]), np.zeros(2)) == 5.0
    y = np.array([1.0, np.nan])
    assert not (o.normwise_err(y, np.ones(2)) < 1e30)


# ------------------------------------------------------------------ ternariser
#
# The offline step: W' = W R_K^T, then per 128-group a threshold search over
# c_j mean|w|, c_j = (j + 1) / 32, with the least-squares scale of each
# candidate's trits rounded to fp16 and the least reconstruction error winning.

def pin_f16_rounding_is_single(o, read_golden=None):
    """The scale is rounded once, float64 -> fp16, to nearest even (no stop at fp32)."""
    cases = [
        (1.0 + 2.0 ** -11 + 2.0 ** -40, 1.0 + 2.0 ** -10),  # above the tie: up (via fp32: 1.0)
        (1.0 + 2.0 ** -11, 1.0),                           # tie: to even
        (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),           # tie: to even, up
        (65519.99, 65504.0), (65520.0, np.inf),            # the top of the range
        (2.0 ** -25, 0.0), (2.0 ** -25 + 2.0 ** -45, 2.0 ** -24),  # subnormal tie / just above
        (3 * 2.0 ** -25, 2.0 ** -23), (0.0, 0.0),
    ]
    for v, want in cases:
        got = o.f64_to_f16_bits(np.array([v])).view(np.float16).astype(np.float64)[0]
        assert got == want, (v, got, want)


def _one_group(o, w):
    t, s, j, bad = o.ternarize(np.asarray(w, dtype=np.float64).reshape(1, 128))
    return t[0], float(s.view(np.float16).astype(np.float64)[0, 0]), int(j[0, 0]), bad


def pin_ternarize_hand_blocks(o, read_golden=None):
    signs = np.where(np.arange(128) % 3 == 0, -1.0, 1.0)
    # equal magnitudes: every threshold up to 0.5 keeps all, error 0 -> the first candidate
    t, s, j, bad = _one_group(o, 0.5 * signs)
    assert (t == signs).all() and s == 0.5 and j == 0 and bad == 0
    # 16 weights of 1 among 112 of 0.01: a = (16 + 1.12) / 128 = 0.13375; the first
    # threshold above 0.01 is 3/32 a = 0.01254 (j = 2), which keeps exactly the 16
    w = np.full(128, 0.01)
    w[::8] = 1.0
    t, s, j, bad = _one_group(o, w * signs)
    assert j == 2 and s == 1.0 and bad == 0
    assert (t == np.where(w == 1.0, signs, 0)).all()
    # all zero: zero trits, scale 0, not bad
    t, s, j, bad = _one_group(o, np.zeros(128))
    assert (t == 0).all() and s == 0.0 and j == -1 and bad == 0
    # non-finite weight, or a scale beyond fp16: bad, stored as zeros
    for v in (np.nan, np.inf):
        w = np.full(128, 0.5)
        w[7] = v
        t, s, j, bad = _one_group(o, w)
        assert (t == 0).all() and s == 0.0 and bad == 1
    # a candidate whose scale overflows fp16 has infinite error: for equal weights of 1e6
    # only the thresholds above them (c_j > 1, nothing kept, scale 0) are finite
    t, s, j, bad = _one_group(o, np.full(128, 1e6))
    assert (t == 0).all() and s == 0.0 and j == 32 and bad == 0
    # one weight of 1e6 is kept by every threshold (2 a < 1e6), so every candidate overflows
    w = np.zeros(128)
    w[3] = 1e6
    t, s, j, bad = _one_group(o, w)
    assert (t == 0).all() and s == 0.0 and bad == 1
    # 65504 is the largest finite fp16: kept
    t, s, j, bad = _one_group(o, np.full(128, 65504.0))
    assert (t == 1).all() and s == 65504.0 and bad == 0


def _ternarize_by_sorting(w):
    """Independent search: sort the magnitudes, count each threshold's keepers by
    bisection, and take the error from prefix sums, E = sum w^2 - 2 s P + n s^2."""
    import math
    m = np.abs(w)
    desc = np.sort(m)[::-1]
    prefix = np.concatenate([[0.0], np.cumsum(desc)])
    total = math.fsum(m * m)
    a = math.fsum(m) / 128
    best = None
    for j in range(64):
        theta = (j + 1) / 32 * a
        cnt = int(np.searchsorted(-desc, -theta, side="right"))   # magnitudes >= theta
        s = prefix[cnt] / cnt if cnt else 0.0
        s16 = float(np.float16(s))
        e = total - 2 * s16 * prefix[cnt] + cnt * s16 * s16
        if best is None or e < best[0] - 1e-12 * total:
            best = (e, j, s16, theta)
    e, j, s16, theta = best
    return np.where(m >= theta, np.sign(w), 0).astype(np.int8), s16, j


def pin_ternarize_matches_sorted_search(o, read_golden=None):
    g = np.random.default_rng(20)
    groups = [g.standard_normal(128), g.laplace(size=128) * 1e-3, g.standard_t(3, size=128),
              np.abs(g.standard_normal(128)), g.standard_normal(128) * 2.0 ** 12]
    # dyadic magnitudes k/64 with sum 64, so a = 1/2 and every threshold (j+1)/64 equals
    # some magnitude: the >= of the threshold rule decides every candidate
    k = np.full(128, 32)
    d = g.integers(-31, 32, size=64)
    k[:64] += d
    k[64:] -= d
    groups.append(k / 64 * np.where(g.integers(0, 2, 128) == 1, -1.0, 1.0))
    sparse = np.zeros(128)
    sparse[g.choice(128, 5, replace=False)] = g.standard_normal(5)
    groups.append(sparse)
    for w in groups:
        t, s, j, bad = _one_group(o, w)
        t2, s2, j2 = _ternarize_by_sorting(w)
        assert bad == 0 and j == j2 and s == s2 and (t == t2).all(), (j, j2, s, s2)


def pin_ternarize_invariances(o, read_golden=None):
    g = np.random.default_rng(21)
    w = g.standard_normal((6, 256))
    t, s, j, _ = o.ternarize(w)
    for p2 in (2.0 ** 5, 2.0 ** -5):           # a power of two moves the scale, not the trits
        t2, s2, j2, _ = o.ternarize(w * p2)
        assert (t2 == t).all() and (j2 == j).all()
        assert (s2.view(np.float16).astype(float) == s.view(np.float16).astype(float) * p2).all()
    t2, s2, j2, _ = o.ternarize(-w)             # negation flips the trits only
    assert (t2 == -t).all() and (s2 == s).all()
    perm = np.concatenate([g.permutation(128), 128 + g.permutation(128)])
    t2, s2, _, _ = o.ternarize(w[:, perm])      # a permutation inside each group permutes the trits
    assert (t2 == t[:, perm]).all() and (s2 == s).all()


def pin_ternarize_gaussian_distortion(o, read_golden=None):
    """The best three-level quantiser of N(0, 1) (Max, 1960) has thresholds +-0.612,
    levels +-1.224 and mean squared error 0.1902; a per-group fitted search can only
    come in at or just under it, with thresholds near 0.612 sigma."""
    g = np.random.default_rng(22)
    w = g.standard_normal((64, 2048))
    t, s, j, bad = o.ternarize(w)
    what = t * np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)
    mse = np.mean((what - w) ** 2)
    assert bad == 0 and 0.175 < mse < 0.1902, mse
    a = np.mean(np.abs(w).reshape(-1, 128), axis=1)
    thr = (j.ravel() + 1) / 32 * a
    assert 0.55 < np.median(thr) < 0.67, np.median(thr)
    lv = s.view(np.float16).astype(np.float64)
    assert 1.15 < np.median(lv) < 1.30, np.median(lv)


def pin_rotate_weights_identity(o, read_golden=None):
    """W x = (W R_K^T)(R_K x) for every x: the rotated weights act on rotated inputs."""
    g = np.random.default_rng(23)
    sb = g.integers(0, 2 ** 32, size=64, dtype=np.uint64).astype(np.uint32)
    w = g.standard_normal((12, 2048))
    x = g.standard_normal((3, 2048))
    lhs = o.rotate_weights(w, sb) @ o.rotate(x, sb).T
    assert np.max(np.abs(lhs - w @ x.T)) < 1e-10


def pin_quantize_tracks_fp_product(o, read_golden=None):
    """y = W_hat (R x) against W x: Gaussian weights give the quantiser's own error
    (sqrt 0.187); weights with 1 % outlier columns x20 stay there in the rotated basis,
    and ternarising them unrotated is more than twice as bad in squared error."""
    g = np.random.default_rng(24)
    sb = g.integers(0, 2 ** 32, size=64, dtype=np.uint64).astype(np.uint32)
    w = g.standard_normal((64, 2048))
    cols = g.choice(2048, 20, replace=False)
    w_out = w.copy()
    w_out[:, cols] *= 20.0
    x = g.standard_normal((32, 2048))
    for ww, lo, hi in ((w, 0.40, 0.46), (w_out, 0.38, 0.46)):
        t, s, _, bad = o.quantize_weights(ww, sb)
        what = t * np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)
        e = o.normwise_err(o.rotate(x, sb) @ what.T, x @ ww.T)
        assert bad == 0 and lo < e < hi, e
    t, s, _, _ = o.ternarize(w_out)
    what = t * np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)
    e_unrot = o.normwise_err(x @ what.T, x @ w_out.T)
    assert e_unrot ** 2 > 2 * 0.46 ** 2, e_unrot


ALL_PINS = [
    pin_base3_page_example, pin_base3_bijection, pin_base3_pad_and_size, pin_base3_bad_counts,
    pin_2bit_base4_number, pin_2bit_bijection, pin_2bit_bad_counts, pin_bits_per_weight,
    pin_hadamard_page_h4, pin_hadamard_sylvester, pin_rotation_orthogonal,
    pin_rotation_closed_forms, pin_rotation_butterfly, pin_rotation_inverse,
    pin_gemv_bruteforce, pin_gemv_associativity, pin_gemv_unit_inputs,
    pin_gemv_zero_and_linearity, pin_gemm_rows_are_gemv,
    pin_rel_err_hand_cases, pin_normwise_err_hand_cases,
    pin_f16_rounding_is_single, pin_ternarize_hand_blocks, pin_ternarize_matches_sorted_search,
    pin_ternarize_invariances, pin_ternarize_gaussian_distortion, pin_rotate_weights_identity,
    pin_quantize_tracks_fp_product,
]
