"""Seeded random shapes through every product entry point, against the oracle.

The fixed-shape tests pin the workloads and the edges each kernel was written for; this sweep
draws shapes that none of them picks (row counts that leave any number of row tiles in the last
workgroup, K anywhere from one block to seventeen, batches 1..32, both packings, every activation
type), so each launch plan the library can choose runs on shapes nobody tuned it for.  Every case
is named before its GPU step; inputs come from the seeded generators, expected values from the
oracle only.
"""
import numpy as np
import pytest
import torch

import fwht_rotation_sqrt_amd as tb
import oracle
import synth
from gpu_util import TOL, act_dev, dev, host, note, scales_dev, signs_dev

pytestmark = pytest.mark.gpu

PACK = {"2bit": oracle.pack_2bit, "base3": oracle.pack_base3}
SWEEP_SEED = 0x5EED


def _cases(count, seed):
    g = np.random.Generator(np.random.Philox(seed))
    out = []
    for i in range(count):
        packing = ("2bit", "base3")[int(g.integers(2))]
        blocks = int(g.integers(1, 18))                     # K = 1024 .. 17408
        k = 1024 * blocks
        # rows: log-uniform from 1 to ~48 M weights per case, or in the upper half of that range
        # (so both a ragged single tile and many tiles per workgroup come up)
        nmax = max(2, min(40000, 48_000_000 // k))
        n = int(np.exp(g.uniform(0.0, np.log(nmax)))) if g.integers(3) else int(g.integers(nmax // 2, nmax))
        b = int(g.choice([1, 1, 1, 2, 3, 5, 8, 9, 13, 32]))
        x_dtype = ("f32", "f16", "bf16")[int(g.integers(3))]
        out.append((i, packing, n, k, b, x_dtype))
    return out


def _inputs(i, packing, n, k, b, x_dtype):
    g = synth.rng(280, 0, i, k // 1024)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x32 = g.standard_normal((b, k)).astype(np.float32)
    if x_dtype == "bf16":
        xbits = synth.f32_to_bf16_bits(x32)
        x64, xd = synth.bf16_bits_to_f64(xbits), act_dev(xbits, "bf16")
    elif x_dtype == "f16":
        x16 = x32.astype(np.float16)
        x64, xd = x16.astype(np.float64), dev(x16)
    else:
        x64, xd = x32.astype(np.float64), dev(x32)
    packed, _ = PACK[packing](t)
    return packed, s, signs, x64, xd


@pytest.mark.parametrize("case", _cases(48, SWEEP_SEED), ids=lambda c: f"{c[1]}-n{c[2]}-k{c[3]}-b{c[4]}-{c[5]}")
def test_sweep_linear_entry_points(case):
    """tb_linear, tb_linear_ws (workspace filled with NaN first) and tb_gemv on the exact x'
    (fp32), every batch row against the oracle: every weight row up to 8 M weights, else every
    7th row and the first and last 32."""
    i, packing, n, k, b, x_dtype = case
    note(f"sweep {packing} n={n} k={k} b={b} x={x_dtype}")
    packed, s, signs, x64, xd = _inputs(*case)
    xr = oracle.rotate(x64, signs)
    rows = np.arange(n) if n * k <= 8_000_000 else \
        np.unique(np.concatenate([np.arange(0, n, 7), np.arange(32), np.arange(n - 32, n)]))
    want = oracle.gemv(packing, packed[rows], s[rows], xr, k)
    pd, sd, sgn = dev(packed), scales_dev(s), signs_dev(signs)
    got = host(tb.tb_linear(packing, pd, sd, xd, sgn))
    assert oracle.rel_err(got[:, rows], want) < TOL, "tb_linear"
    need = tb.tb_linear_workspace_bytes(packing, b, n, k)
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    got = host(tb.tb_linear_ws(packing, pd, sd, xd, sgn, workspace=ws))
    assert oracle.rel_err(got[:, rows], want) < TOL, "tb_linear_ws"
    got = host(tb.tb_gemv(packing, pd, sd, dev(xr.astype(np.float32))))
    assert oracle.rel_err(got[:, rows], want) < TOL, "tb_gemv"


def _gemm_cases(count, seed):
    g = np.random.Generator(np.random.Philox(seed))
    out = []
    for i in range(count):
        packing = ("2bit", "base3")[int(g.integers(2))]
        m = int(g.integers(1, 400))
        n = int(g.integers(1, 1200))
        k = 128 * int(g.integers(1, 24))
        out.append((i, packing, m, n, k))
    return out


@pytest.mark.parametrize("case", _gemm_cases(16, SWEEP_SEED + 1), ids=lambda c: f"{c[1]}-m{c[2]}-n{c[3]}-k{c[4]}")
def test_sweep_gemm(case):
    """tb_gemm at random M (both sides of the 96-row switch), N and K (any number of groups)."""
    i, packing, m, n, k = case
    note(f"sweep gemm {packing} m={m} n={n} k={k}")
    g = synth.rng(281, 0, i, k // 128)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    xr = g.standard_normal((m, k)).astype(np.float16)
    packed, _ = PACK[packing](t)
    want = oracle.gemm(packing, packed, s, xr.astype(np.float64), k)
    got = host(tb.tb_gemm(packing, dev(packed), scales_dev(s), dev(xr)))
    assert oracle.rel_err(got, want) < TOL
