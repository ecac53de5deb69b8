"""Persistent multi-linear decode (tb_decode_chain) against the oracle's own chain.

Linear i > 0 of a chain reads the first K outputs of linear i - 1, so every
linear's input depends on the previous output.  The oracle runs the same chain
in fp64 from the same seeded weights and x0 (its inputs come from its own
previous outputs, never from the GPU's); every output meets the row-rms
relative error bound.
"""
import numpy as np
import pytest
import torch

import fwht_rotation_sqrt_amd as tb
import oracle
import synth
from gpu_util import TOL, act_dev, dev, host, note, scales_dev, signs_dev

pytestmark = pytest.mark.gpu


def _chain_inputs(wid, ns, k):
    lins = []
    for i, n in enumerate(ns):
        g = synth.rng(wid, synth.T_TRITS, 0, i)
        t = synth.trits(g, n, k)
        s = synth.scales_f16(synth.rng(wid, synth.T_SCALES, 0, i), n, k)
        packed, _ = oracle.pack_base3(t)
        lins.append((packed, s))
    signs = synth.sign_bits(synth.rng(wid, synth.T_SIGNS), k)
    x0 = synth.activations(synth.rng(wid, synth.T_X), 1, k, dtype="bf16")
    return lins, signs, x0


def _oracle_chain(lins, signs, x0, k, rows_last=None):
    """y_0 = W_0 (R x0); y_i = W_i (R y_{i-1}[:K]); the last linear on rows_last only (if given)."""
    x = synth.bf16_bits_to_f64(x0)[0]
    outs = []
    for i, (packed, s) in enumerate(lins):
        last = i == len(lins) - 1
        rows = rows_last if (last and rows_last is not None) else np.arange(packed.shape[0] if last else k)
        y = oracle.gemv("base3", packed[rows], s[rows], oracle.rotate(x[None], signs), k)[0]
        outs.append((rows, y))
        if not last:
            x = y[:k]
    return outs


def _run(lins, signs, x0, sync, spin_limit=0):
    linears = [(dev(p), scales_dev(s)) for p, s in lins]
    return tb.tb_decode_chain("base3", linears, act_dev(x0, "bf16")[0], signs_dev(signs), sync,
                              spin_limit=spin_limit)


def _check(outs_gpu, outs_ref):
    for i, ((rows, want), got) in enumerate(zip(outs_ref, outs_gpu)):
        g = host(got)[rows]
        err = oracle.rel_err(g[None], want[None])
        note(f"  linear {i}: {len(rows)} rows checked, rel err {err:.2e}")
        assert err < TOL, (i, err)


def test_chain_dependent_linears_small():
    """Three dependent linears at K = 2048 (ragged last tile), then the same sync buffer again for
    a two-linear chain at K = 1024: the counts the first call leaves must be zero."""
    sync = torch.zeros(tb.TB_CHAIN_MAX + 2, dtype=torch.int32, device="cuda")
    for wid, ns, k in ((310, (4096, 2048, 3001), 2048), (311, (1024, 777), 1024)):
        note(f"chain K={k} N={ns}")
        lins, signs, x0 = _chain_inputs(wid, ns, k)
        outs = _run(lins, signs, x0, sync)
        _check(outs, _oracle_chain(lins, signs, x0, k))
        assert (host(sync) == 0).all()


def test_chain_token_layer_full_size():
    """One layer of the 27B token stream as one launch: q/k/v (15360 x 5120), o (5120 x 5120) and
    gate/up (34816 x 5120, more row tiles per compute unit than one round holds), each reading the
    previous output; the last linear checked on sampled rows."""
    H, F = synth.HIDDEN, synth.FFN
    ns = (3 * H, H, 2 * F)
    note(f"chain token layer N={ns}")
    lins, signs, x0 = _chain_inputs(312, ns, H)
    sync = torch.zeros(len(ns) + 2, dtype=torch.int32, device="cuda")
    outs = _run(lins, signs, x0, sync)
    rows = np.unique(np.concatenate([[0, 1, 2 * F - 1], synth.rng(312, 9).integers(0, 2 * F, 61)]))
    _check(outs, _oracle_chain(lins, signs, x0, H, rows))
    # a second call reuses the sync buffer and gives the same outputs
    again = _run(lins, signs, x0, sync)
    for a, b in zip(outs, again):
        assert oracle.rel_err(host(b)[None], host(a)[None]) < TOL


def test_chain_wait_times_out_cleanly():
    """A count that never arrives (forced from the host: word 0 starts far below zero) ends every
    wait after spin_limit polls: the launch finishes, the status bit is set and the counts are
    cleared; a cleared buffer then works again."""
    ns, k = (2048, 1024), 1024
    lins, signs, x0 = _chain_inputs(313, ns, k)
    sync = torch.zeros(len(ns) + 2, dtype=torch.int32, device="cuda")
    sync[0] = -(1 << 30)
    note("chain forced time-out")
    _run(lins, signs, x0, sync, spin_limit=64)
    s = host(sync)
    assert s[len(ns) + 1] & 1
    sync.zero_()
    outs = _run(lins, signs, x0, sync)
    _check(outs, _oracle_chain(lins, signs, x0, k))
    assert (host(sync) == 0).all()
