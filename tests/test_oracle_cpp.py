"""The plain C++ oracle agrees with the pinned numpy oracle and with a closed form (CPU only)."""
import numpy as np
import pytest

import oracle
import synth
from oracle import cpp_oracle


@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("b,n,k", [(1, 5, 1024), (3, 37, 2048), (2, 16, 5120)])
def test_cpp_oracle_matches_numpy_oracle(packing, b, n, k):
    g = synth.rng(280, 0, n, k // 1024)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x = g.standard_normal((b, k))
    packed, _ = (oracle.pack_2bit if packing == "2bit" else oracle.pack_base3)(t)
    want = oracle.gemv(packing, packed, s, oracle.rotate(x, signs), k)
    for threads in (1, 3):
        got = cpp_oracle.linear(packing, packed, s, x, signs, threads)
        assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    # x already rotated
    got = cpp_oracle.linear(packing, packed, s, oracle.rotate(x, signs), None)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_cpp_oracle_unit_rotated_input(packing):
    """x = R^T e_j (so that R x = e_j exactly in fp64: S H e_j / 32 is +-1/32)
    picks one weight: y[n] = s[n][j / 128] t[n][j]."""
    n, k = 9, 2048
    g = synth.rng(281, 0, 0, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    packed, _ = (oracle.pack_2bit if packing == "2bit" else oracle.pack_base3)(t)
    sv = synth.f16_bits_to_f64(s)
    for j in (0, 5, 1023, 1024, 1500, 2047):
        blk, jj = divmod(j, 1024)
        col = np.array([(-1.0) ** bin(i & jj).count("1") for i in range(1024)])
        x = np.zeros((1, k))
        x[0, 1024 * blk:1024 * (blk + 1)] = oracle.sign_vector(signs, k)[1024 * blk:1024 * (blk + 1)] * col / 32
        y = cpp_oracle.linear(packing, packed, s, x, signs)
        assert np.array_equal(y[0], sv[:, j // 128] * t[:, j])


def test_cpp_oracle_rejects_bad_sizes():
    with pytest.raises(ValueError):
        cpp_oracle.linear("base3", np.zeros((2, 26), np.uint8), np.zeros((2, 1), np.uint16), np.zeros((1, 128)),
                          np.zeros(4, np.uint32))      # K = 128 cannot be rotated by 1024-blocks


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_cpp_pack_unpack_match_numpy_oracle(packing):
    """The C++ packings against the pinned numpy ones, invalid inputs included: trits outside
    {-1, 0, 1}; 2-bit code 11; base-3 bytes >= 243 and last bytes with pad digits other than 1."""
    g = synth.rng(282, 0, 0, 0)
    t = synth.trits(g, 7, 1024)
    t[1, 5] = 3
    t[4, 700] = -2
    want, bad = (oracle.pack_2bit if packing == "2bit" else oracle.pack_base3)(t)
    got, gbad = cpp_oracle.pack(packing, t)
    assert np.array_equal(got, want) and gbad == bad == 2
    p = want.copy()
    if packing == "2bit":
        p[0, 3] |= 0xC0            # one code 11
        p[6, 200] = 0xFF           # four codes 11
    else:
        p[0, 3] = 250              # not a code
        p[2, 25] = 108 + 81        # last byte of group 0: pad digit 4 = 2
        p[5, 26 + 25] = 134 - 27   # last byte of group 1: pad digit 3 = 0
    want_t, want_bad = (oracle.unpack_2bit if packing == "2bit" else oracle.unpack_base3)(p, 1024)
    got_t, got_bad = cpp_oracle.unpack(packing, p, 1024)
    assert np.array_equal(got_t, want_t) and got_bad == want_bad and want_bad >= 3
