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


ALL_PINS = [
    pin_base3_page_example, pin_base3_bijection, pin_base3_pad_and_size, pin_base3_bad_counts,
    pin_2bit_base4_number, pin_2bit_bijection, pin_2bit_bad_counts, pin_bits_per_weight,
    pin_hadamard_page_h4, pin_hadamard_sylvester, pin_rotation_orthogonal,
    pin_rotation_closed_forms, pin_rotation_butterfly, pin_rotation_inverse,
    pin_gemv_bruteforce, pin_gemv_associativity, pin_gemv_unit_inputs,
    pin_gemv_zero_and_linearity, pin_gemm_rows_are_gemv,
    pin_rel_err_hand_cases, pin_normwise_err_hand_cases,
]
