"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Inputs come from the seeded generator; expected values come only from the
oracle.  Packing and unpacking are bit-exact; products meet the row-rms
relative error bound TOL = 2e-3 (fp32 accumulation against fp64).
"""
import numpy as np
import pytest
import torch

import fwht_rotation_sqrt_amd as tb
import oracle
import synth
from gpu_util import TOL, act_dev, act_f64, dev, f16_ulp_distance, host, note, scales_dev, signs_dev

pytestmark = pytest.mark.gpu

PACK_REF = {"2bit": oracle.pack_2bit, "base3": oracle.pack_base3}
PACK_GPU = {"2bit": tb.tb_pack_2bit, "base3": tb.tb_pack_base3}


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("n,k", [(1, 128), (3, 1024), (37, 5120), (5, 17408), (17408, 5120)])
def test_pack_unpack_bitexact(packing, n, k):
    note(f"pack/unpack {packing} n={n} k={k}")
    t = synth.trits(synth.rng(200, 0, n % 251, k // 128), n, k)
    ref, bad = PACK_REF[packing](t)
    assert bad == 0
    bad_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = PACK_GPU[packing](dev(t), bad_count=bad_d)
    assert np.array_equal(host(packed), ref)
    assert int(host(bad_d)[0]) == 0
    back = tb.tb_unpack(packing, packed, k, bad_count=bad_d)
    assert np.array_equal(host(back), t)
    assert int(host(bad_d)[0]) == 0


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_pack_invalid_inputs_counted(packing):
    note(f"pack invalid {packing}")
    n, k = 4, 256
    t = synth.trits(synth.rng(201, 0), n, k)
    t[0, 3] = 2
    t[2, 100] = -7
    t[3, 255] = 5
    ref, bad = PACK_REF[packing](t)
    assert bad == 3
    bad_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = PACK_GPU[packing](dev(t), bad_count=bad_d)
    assert np.array_equal(host(packed), ref) and int(host(bad_d)[0]) == 3


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_unpack_invalid_codes_counted(packing):
    note(f"unpack invalid {packing}")
    n, k = 3, 384
    t = synth.trits(synth.rng(202, 0), n, k)
    p, _ = PACK_REF[packing](t)
    if packing == "2bit":
        p[0, 5] = 0xFF          # four 11 codes
        p[2, 90] = 0x3C         # two 11 codes
    else:
        p[0, 5] = 250           # >= 243
        p[1, 25] = 95           # last byte of group 0 with pad digits (0, 1)
        p[2, 51] = 243
    want, bad = (oracle.unpack_2bit if packing == "2bit" else oracle.unpack_base3)(p, k)
    bad_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = tb.tb_unpack(packing, dev(p), k, bad_count=bad_d)
    assert np.array_equal(host(got), want)
    assert int(host(bad_d)[0]) == bad and bad > 0


# ------------------------------------------------------------------ rotation

@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,k", [(1, 1024), (1, 5120), (3, 17408), (512, 5120)])
def test_rotate_fp32_out(x_dtype, rows, k):
    note(f"rotate {x_dtype}->f32 rows={rows} k={k}")
    g = synth.rng(210, 0, rows % 251, k // 1024)
    oc = synth.outlier_channels(g, k)
    x = synth.activations(g, rows, k, oc, x_dtype)
    sb = synth.sign_bits(synth.rng(210, synth.T_SIGNS), k)
    want = oracle.rotate(act_f64(x, x_dtype), sb)
    got = host(tb.tb_fwht_rotate(act_dev(x, x_dtype), signs_dev(sb), torch.float32)).astype(np.float64)
    scale = np.sqrt(np.mean(want * want, axis=1, keepdims=True))
    assert np.max(np.abs(got - want) / scale) < 2e-6


@pytest.mark.parametrize("rows,k", [(1, 5120), (512, 5120), (7, 17408)])
def test_rotate_fp16_out_within_one_ulp(rows, k):
    note(f"rotate bf16->f16 rows={rows} k={k}")
    g = synth.rng(211, 0, rows % 251, k // 1024)
    x = synth.activations(g, rows, k, synth.outlier_channels(g, k), "bf16")
    sb = synth.sign_bits(synth.rng(211, synth.T_SIGNS), k)
    want = oracle.rotate(act_f64(x, "bf16"), sb).astype(np.float16)   # round to nearest even
    got = host(tb.tb_fwht_rotate(act_dev(x, "bf16"), signs_dev(sb), torch.float16))
    d = f16_ulp_distance(got, want)
    assert d.max() <= 1
    assert np.mean(d) < 1e-3


def test_rotate_in_place_and_fp16_input():
    note("rotate in place f32 and f16->f32")
    k, rows = 2048, 5
    g = synth.rng(212, 0)
    x = synth.activations(g, rows, k, None, "f32")
    sb = synth.sign_bits(synth.rng(212, synth.T_SIGNS), k)
    want = oracle.rotate(x.astype(np.float64), sb)
    xd = dev(x)
    tb.tb_fwht_rotate(xd, signs_dev(sb), out=xd)
    assert np.max(np.abs(host(xd) - want)) < 1e-5
    x16 = x.astype(np.float16)
    want16 = oracle.rotate(x16.astype(np.float64), sb)
    got = host(tb.tb_fwht_rotate(dev(x16), signs_dev(sb), torch.float32))
    assert np.max(np.abs(got - want16)) < 1e-5


# ------------------------------------------------------------------ decode product

def _linear(wid, n, k, rows, x_dtype, outliers, layer=0, linear=0):
    li = synth.linear_inputs(wid, n, k, rows, x_dtype, outliers, layer, linear)
    return li


@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("n,k", [(1, 128), (3, 1024), (16, 1024), (37, 2048), (130, 5120), (1000, 1024),
                                 (7, 640), (50, 1152), (300, 3200), (81, 17408)])
@pytest.mark.parametrize("xr_dtype", [torch.float32, torch.float16])
def test_gemv_small_shapes(packing, n, k, xr_dtype):
    note(f"gemv {packing} n={n} k={k} xr={xr_dtype}")
    g = synth.rng(220, 0, n % 251, k // 128)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    xr = g.standard_normal((8, k)).astype(np.float32)
    if xr_dtype == torch.float16:
        xr = xr.astype(np.float16)
    packed, _ = PACK_REF[packing](t)
    want = oracle.gemv(packing, packed, s, xr.astype(np.float64), k)
    pd, sd, xd = dev(packed), scales_dev(s), dev(xr)
    for b in (1, 2, 5, 8):
        got = host(tb.tb_gemv(packing, pd, sd, xd[:b].contiguous()))
        assert got.shape == (b, n)
        assert oracle.rel_err(got, want[:b]) < TOL


def _e2e_gemv(wid, packing, n, k, x_dtype, outliers, batches, layer=0, linear=0):
    li = _linear(wid, n, k, max(batches), x_dtype, outliers, layer, linear)
    ref_packed, _ = PACK_REF[packing](li.trits)
    packed = PACK_GPU[packing](dev(li.trits))
    assert np.array_equal(host(packed), ref_packed)
    x64 = act_f64(li.x, x_dtype)
    want = oracle.gemv(packing, ref_packed, li.scales, oracle.rotate(x64, li.signs), k)
    sd, sgn, xd = scales_dev(li.scales), signs_dev(li.signs), act_dev(li.x, x_dtype)
    errs = {}
    for b in batches:
        xr = tb.tb_fwht_rotate(xd[:b].contiguous(), sgn, torch.float32)
        y = host(tb.tb_gemv(packing, packed, sd, xr))
        errs[b] = oracle.rel_err(y, want[:b])
        assert errs[b] < TOL, (b, errs[b])
        if k % 1024 == 0:
            # the same linear with the rotation inside the product
            y1 = host(tb.tb_linear(packing, packed, sd, xd[:b].contiguous(), sgn))
            e1 = oracle.rel_err(y1, want[:b])
            assert e1 < TOL, ("tb_linear", b, e1)
            # one pass over the weights at any batch, x' through a workspace
            y2 = host(tb.tb_linear_ws(packing, packed, sd, xd[:b].contiguous(), sgn))
            e2 = oracle.rel_err(y2, want[:b])
            assert e2 < TOL, ("tb_linear_ws", b, e2)
    return errs


def test_linear1024_2bit_b1_end_to_end():
    note("1024x1024 2-bit batch 1, fp32 activations")
    _e2e_gemv(0, "2bit", 1024, 1024, "f32", False, (1,))


def test_gemv_ffn_base3_b1_end_to_end():
    note("17408x5120 base-3 batch 1, bf16 activations with outliers")
    _e2e_gemv(1, "base3", synth.FFN, synth.HIDDEN, "bf16", True, (1,))


@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("li", range(len(synth.BLOCK_LINEARS)), ids=[l.name for l in synth.BLOCK_LINEARS])
def test_block_linears_b1_b8_b32(packing, li):
    """Every block linear at full size, batch 1 and 8 (limb kernel) and 32
    (one-pass batched kernel for tb_gemv, chunks of 8 for tb_linear)."""
    lin = synth.BLOCK_LINEARS[li]
    note(f"block linear {lin.name} {lin.n}x{lin.k} {packing} batch 1, 8 and 32")
    _e2e_gemv(2, packing, lin.n, lin.k, "bf16", False, (1, 8, 32), 0, li)


@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("n,k", [(1, 1024), (16, 1024), (37, 2048), (300, 3072), (1000, 5120), (81, 17408)])
@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_linear_fused_rotation(packing, n, k, x_dtype):
    note(f"tb_linear {packing} n={n} k={k} x={x_dtype}")
    g = synth.rng(240, 0, n % 251, k // 1024)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x32 = g.standard_normal((8, k)).astype(np.float32)
    if x_dtype == "bf16":
        xbits = synth.f32_to_bf16_bits(x32)
        x64, xd = synth.bf16_bits_to_f64(xbits), act_dev(xbits, "bf16")
    elif x_dtype == "f16":
        x16 = x32.astype(np.float16)
        x64, xd = x16.astype(np.float64), dev(x16)
    else:
        x64, xd = x32.astype(np.float64), dev(x32)
    packed, _ = PACK_REF[packing](t)
    want = oracle.gemv(packing, packed, s, oracle.rotate(x64, signs), k)
    pd, sd, sgn = dev(packed), scales_dev(s), signs_dev(signs)
    for b in (1, 3, 5, 8):
        got = host(tb.tb_linear(packing, pd, sd, xd[:b].contiguous(), sgn))
        assert got.shape == (b, n)
        assert oracle.rel_err(got, want[:b]) < TOL, b


@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("exp2", [-120, 100])
def test_gemv_extreme_magnitudes(packing, exp2):
    """Activations scaled by 2^exp2 (exactly), at every product path: the limb
    kernels (batch 1..8; at 2^-120 every group's power-of-two scale hits its
    upper clamp, at 2^100 it is far negative) and the fp16 matrix-core kernel
    (batch 6/9..32), whose per-row-and-group power-of-two scale brings x'
    into the fp16 range first.  The error bound is relative to the row rms,
    so it is the same at any scale."""
    n, k = 300, 5120
    note(f"gemv/linear {packing} x * 2^{exp2}")
    g = synth.rng(250, 0, exp2 & 255, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x32 = np.ldexp(g.standard_normal((tb.TB_GEMV_MAX_BATCH, k)), exp2).astype(np.float32)
    assert np.all(np.isfinite(x32)) and np.min(np.abs(x32[x32 != 0])) > 0
    x64 = x32.astype(np.float64)
    packed, _ = PACK_REF[packing](t)
    pd, sd, xd, sgn = dev(packed), scales_dev(s), dev(x32), signs_dev(signs)
    # x' given: the exact rotation of the fp32 activations, rounded to fp32
    xr = oracle.rotate(x64, signs)
    want = oracle.gemv(packing, packed, s, xr, k)
    xrd = dev(xr.astype(np.float32))
    for b in (1, 4, 6, 8, 9, 17, tb.TB_GEMV_MAX_BATCH):
        got = host(tb.tb_gemv(packing, pd, sd, xrd[:b].contiguous()))
        assert oracle.rel_err(got, want[:b]) < TOL, ("tb_gemv", b)
        # rotation fused, or through the workspace
        got = host(tb.tb_linear(packing, pd, sd, xd[:b].contiguous(), sgn))
        assert oracle.rel_err(got, want[:b]) < TOL, ("tb_linear", b)
        got = host(tb.tb_linear_ws(packing, pd, sd, xd[:b].contiguous(), sgn))
        assert oracle.rel_err(got, want[:b]) < TOL, ("tb_linear_ws", b)


@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("n,k", [(1, 128), (16, 1024), (37, 1152), (300, 3200), (1000, 5120), (81, 17408),
                                 (5000, 1024)])
@pytest.mark.parametrize("xr_dtype", [torch.float32, torch.float16])
def test_gemv_batches_9_to_32_one_pass(packing, n, k, xr_dtype):
    """tb_gemv at 9..32 rows: one pass over the weights on the fp16 matrix
    cores (one or two blocks of 16 rows, ragged row and column tails, 1..5
    row tiles per workgroup, K split over the waves unevenly)."""
    note(f"gemv wide {packing} n={n} k={k} xr={xr_dtype}")
    g = synth.rng(222, 0, n % 251, k // 128)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    xr = g.standard_normal((tb.TB_GEMV_MAX_BATCH, k)).astype(np.float32)
    if xr_dtype == torch.float16:
        xr = xr.astype(np.float16)
    packed, _ = PACK_REF[packing](t)
    want = oracle.gemv(packing, packed, s, xr.astype(np.float64), k)
    pd, sd, xd = dev(packed), scales_dev(s), dev(xr)
    for b in (9, 16, 17, 21, tb.TB_GEMV_MAX_BATCH):
        got = host(tb.tb_gemv(packing, pd, sd, xd[:b].contiguous()))
        assert got.shape == (b, n)
        err = oracle.rel_err(got, want[:b])
        note(f"  b={b} rel err {err:.2e}")
        assert err < TOL, (b, err)


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_gemv_batches_9_to_32_magnitudes(packing):
    """The one-pass path carries fp32 x' as fp16 hi + lo after a power-of-two
    scale per activation row and group: the relative error stays at the fp32
    level at any magnitude, including values past the fp16 range (1e30), far
    below its normal range (2^-20, and 2^-120 with fp32 subnormals), rows of very
    different size in one call, and groups that are all zero."""
    n, k = 300, 2048
    note(f"gemv wide {packing} magnitudes")
    g = synth.rng(223, 0, 0, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    packed, _ = PACK_REF[packing](t)
    pd, sd = dev(packed), scales_dev(s)
    base = g.standard_normal((16, k))
    cases = {
        "near fp16 max": base * (60000.0 / np.abs(base).max()),
        "1e30": base * 1e30,
        "2^-20": np.ldexp(base, -20),
        "2^-120": np.ldexp(base, -120),          # the smallest entries are fp32 subnormals
        "mixed rows": base * np.ldexp(1.0, np.arange(16)[:, None] * 16 - 120),
        "zero groups": base * (np.arange(k)[None, :] // 128 % 3 != 1),
    }
    for name, x in cases.items():
        x32 = x.astype(np.float32)
        want = oracle.gemv(packing, packed, s, x32.astype(np.float64), k)
        got = host(tb.tb_gemv(packing, pd, sd, dev(x32)))
        err = oracle.rel_err(got, want)
        note(f"  {name}: rel err {err:.2e}")
        assert err < 1e-5, (name, err)


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_gemv_linear_batches_above_8(packing):
    """Batches above 8: tb_gemv takes them in one pass, tb_linear as chunks
    of 8 rows over the weights; every row must match the oracle, across
    chunk boundaries and with a ragged last chunk."""
    n, k = 200, 3072
    note(f"gemv/linear {packing} batches 9..32")
    g = synth.rng(260, 0, 0, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x32 = g.standard_normal((tb.TB_GEMV_MAX_BATCH, k)).astype(np.float32)
    x64 = x32.astype(np.float64)
    packed, _ = PACK_REF[packing](t)
    xr = oracle.rotate(x64, signs)
    want = oracle.gemv(packing, packed, s, xr, k)
    pd, sd, sgn = dev(packed), scales_dev(s), signs_dev(signs)
    xrd, xd = dev(xr.astype(np.float32)), dev(x32)
    for b in (9, 16, 21, tb.TB_GEMV_MAX_BATCH):
        got = host(tb.tb_gemv(packing, pd, sd, xrd[:b].contiguous()))
        assert got.shape == (b, n)
        assert oracle.rel_err(got, want[:b]) < TOL, ("tb_gemv", b)
        got = host(tb.tb_linear(packing, pd, sd, xd[:b].contiguous(), sgn))
        assert oracle.rel_err(got, want[:b]) < TOL, ("tb_linear", b)
    # tb_linear_ws: one caller workspace of the largest size, reused by every batch in turn
    ws = torch.empty(tb.tb_linear_workspace_bytes(packing, tb.TB_GEMV_MAX_BATCH, n, k), dtype=torch.uint8,
                     device="cuda")
    for b in (1, 2, 5, 6, 8, 9, 16, 21, tb.TB_GEMV_MAX_BATCH, 7, 1):
        got = host(tb.tb_linear_ws(packing, pd, sd, xd[:b].contiguous(), sgn, workspace=ws))
        assert oracle.rel_err(got, want[:b]) < TOL, ("tb_linear_ws", b)
    need = tb.tb_linear_workspace_bytes(packing, 16, n, k)
    with pytest.raises(tb.TBError, match="workspace"):
        tb.tb_linear_ws(packing, pd, sd, xd[:16].contiguous(), sgn, workspace=ws[:need - 16])


@pytest.mark.parametrize("n,k,x_dtype", [(300, 6144, "f32"), (777, 11264, "f16"), (5120, 17408, "bf16"),
                                         (9000, 17408, "bf16"), (12000, 17408, "f32")])
def test_linear_ws_batch1_rows_in_parts(n, k, x_dtype):
    """Batch 1, base-3, K above 5120 through tb_linear_ws: the row is taken in parts of K by
    separate workgroups (6144: two parts of three blocks; 11264: three of four, the last padded
    by one; 17408, the down projection: four of five, the last padded by three), the partial sums
    go to the workspace (filled with NaN first: every word must be written) and a second launch
    adds them.  9000 rows put nine tiles in a workgroup (one wave per tile); 12000 rows are more
    than the parts' workgroups hold and run as tb_linear.  Sampled rows (every 7th, the first and
    last 16) against the oracle; tb_linear_noalloc gives the same bits."""
    note(f"tb_linear_ws batch 1 base3 n={n} k={k} x={x_dtype}")
    g = synth.rng(275, 0, n % 251, k // 1024)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x32 = g.standard_normal((1, k)).astype(np.float32)
    if x_dtype == "bf16":
        xbits = synth.f32_to_bf16_bits(x32)
        x64, xd = synth.bf16_bits_to_f64(xbits), act_dev(xbits, "bf16")
    elif x_dtype == "f16":
        x16 = x32.astype(np.float16)
        x64, xd = x16.astype(np.float64), dev(x16)
    else:
        x64, xd = x32.astype(np.float64), dev(x32)
    packed, _ = oracle.pack_base3(t)
    rows = np.unique(np.concatenate([np.arange(0, n, 7), np.arange(16), np.arange(n - 16, n)]))
    want = oracle.gemv("base3", packed[rows], s[rows], oracle.rotate(x64, signs), k)
    need = tb.tb_linear_workspace_bytes("base3", 1, n, k)
    assert need == 4 * n * ((k // 1024 + 4) // 5)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    pd, sd, sgn = dev(packed), scales_dev(s), signs_dev(signs)
    got = host(tb.tb_linear_ws("base3", pd, sd, xd, sgn, workspace=ws))
    assert np.isfinite(got).all()
    assert oracle.rel_err(got[:, rows], want) < TOL
    y0 = torch.empty((1, n), dtype=torch.float32, device="cuda")
    assert np.array_equal(host(tb.tb_linear_noalloc("base3", pd, sd, xd, sgn, y0)), got)
    # the same call again on the same workspace: the same bits (the sums run in part order)
    assert np.array_equal(host(tb.tb_linear_ws("base3", pd, sd, xd, sgn, workspace=ws)), got)


@pytest.mark.parametrize("packing,n,k,b,parts", [
    ("base3", 1, 17408, 32, 8),     # one row in a ragged tile, eight parts of 17 groups
    ("2bit", 17, 2048, 16, 2),      # two parts of 8 groups (two parts only from batch 16)
    ("base3", 300, 17408, 9, 8),
    ("base3", 3000, 17408, 8, 6),   # six parts: five of 23 groups, the last of 21
    ("2bit", 5120, 5120, 8, 4),
    ("base3", 9000, 5120, 16, 2),
    ("2bit", 9000, 5120, 9, 1),     # two parts below batch 16 are not taken: whole rows
])
def test_linear_ws_batched_parts_of_k(packing, n, k, b, parts):
    """The batched product in parts of K through tb_linear_ws: where rows are too few for
    five-tile workgroups on every compute unit, P parts of K (at most 8, at least 8 groups each)
    on separate workgroups write their partial sums to the workspace after x' (all filled with NaN
    first: every word must be written) and a second launch adds them in part order.  Every batch
    row against the oracle (every row up to 4 M weights, else every 7th and the first and last 16);
    a repeated call on the same workspace gives the same bits."""
    note(f"tb_linear_ws parts of K {packing} n={n} k={k} b={b} parts={parts}")
    g = synth.rng(276, 0, n % 251, k // 1024)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x = g.standard_normal((b, k)).astype(np.float32)
    packed, _ = PACK_REF[packing](t)
    rows = np.arange(n) if n * k <= 4_000_000 else \
        np.unique(np.concatenate([np.arange(0, n, 7), np.arange(16), np.arange(n - 16, n)]))
    want = oracle.gemv(packing, packed[rows], s[rows], oracle.rotate(x.astype(np.float64), signs), k)
    need = tb.tb_linear_workspace_bytes(packing, b, n, k)
    assert need == 4 * b * k + (4 * parts * b * n if parts > 1 else 0)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    pd, sd, xd, sgn = dev(packed), scales_dev(s), dev(x), signs_dev(signs)
    got = host(tb.tb_linear_ws(packing, pd, sd, xd, sgn, workspace=ws))
    assert np.isfinite(got).all()
    assert oracle.rel_err(got[:, rows], want) < TOL
    assert np.array_equal(host(tb.tb_linear_ws(packing, pd, sd, xd, sgn, workspace=ws)), got)


@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("n", [3 * synth.HIDDEN, 2 * synth.FFN], ids=["qkv_15360", "gate_up_34816"])
def test_concatenated_linears_sampled_rows(packing, n):
    """q/k/v and gate/up as one call each (rows concatenated): 15360 and 34816
    rows of K = 5120, batch 1, 3 and 8, both entry points (34816 rows put 9
    row tiles in a workgroup), and tb_gemv at 9 and 32 rows (one pass).  The
    oracle computes every 13th row and the last 16 (the last, partial
    workgroup)."""
    k = synth.HIDDEN
    note(f"concatenated linear {packing} {n}x{k}")
    g = synth.rng(270, 0, n % 251, 0)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    xbits = synth.f32_to_bf16_bits(g.standard_normal((tb.TB_GEMV_MAX_BATCH, k)).astype(np.float32))
    x64 = synth.bf16_bits_to_f64(xbits)
    ref_packed, _ = PACK_REF[packing](t)
    rows = np.unique(np.concatenate([np.arange(0, n, 13), np.arange(n - 16, n)]))
    xr = oracle.rotate(x64, signs)
    want = oracle.gemv(packing, ref_packed[rows], s[rows], xr, k)
    pd, sd, sgn, xd = dev(ref_packed), scales_dev(s), signs_dev(signs), act_dev(xbits, "bf16")
    xrd = dev(xr.astype(np.float32))
    for b in (1, 3, 8):
        got = host(tb.tb_linear(packing, pd, sd, xd[:b].contiguous(), sgn))
        assert oracle.rel_err(got[:, rows], want[:b]) < TOL, ("tb_linear", b)
        got = host(tb.tb_gemv(packing, pd, sd, xrd[:b].contiguous()))
        assert oracle.rel_err(got[:, rows], want[:b]) < TOL, ("tb_gemv", b)
    for b in (9, tb.TB_GEMV_MAX_BATCH):
        got = host(tb.tb_gemv(packing, pd, sd, xrd[:b].contiguous()))
        assert oracle.rel_err(got[:, rows], want[:b]) < TOL, ("tb_gemv", b)


# ------------------------------------------------------------------ prefill product

@pytest.mark.parametrize("packing", ["2bit", "base3"])
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (5, 37, 1024), (64, 64, 256), (100, 300, 2048), (130, 1000, 5120),
                                   (129, 545, 1152), (7, 273, 640), (32, 300, 2048), (33, 300, 2048),
                                   (96, 300, 2048), (97, 300, 2048), (16, 17408, 5120),
                                   # M > 96 runs on the 128 x 272 tiles: K loops of 1, 2 and 5 groups
                                   (97, 300, 128), (130, 290, 256), (200, 17, 640)])
def test_gemm_small_shapes(packing, m, n, k):
    note(f"gemm {packing} m={m} n={n} k={k}")
    g = synth.rng(230, 0, m % 251, n % 251)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    xr = g.standard_normal((m, k)).astype(np.float16)
    packed, _ = PACK_REF[packing](t)
    want = oracle.gemm(packing, packed, s, xr.astype(np.float64), k)
    got = host(tb.tb_gemm(packing, dev(packed), scales_dev(s), dev(xr)))
    assert oracle.rel_err(got, want) < TOL


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_gemm_pp512_end_to_end(packing):
    note(f"pp512 GEMM M=512 N=17408 K=5120 {packing}, bf16 activations with outliers")
    m, n, k = 512, synth.FFN, synth.HIDDEN
    li = _linear(3, n, k, m, "bf16", True)
    ref_packed, _ = PACK_REF[packing](li.trits)
    packed = (tb.tb_pack_2bit if packing == "2bit" else tb.tb_pack_base3)(dev(li.trits))
    assert np.array_equal(host(packed), ref_packed)
    xr_exact = oracle.rotate(act_f64(li.x, "bf16"), li.signs)
    want = oracle.gemm(packing, ref_packed, li.scales, xr_exact.astype(np.float16).astype(np.float64), k)
    xr = tb.tb_fwht_rotate(act_dev(li.x, "bf16"), signs_dev(li.signs), torch.float16)
    y = host(tb.tb_gemm(packing, packed, scales_dev(li.scales), xr))
    assert oracle.rel_err(y, want) < TOL
    # against the unrounded product too: fp16 rounding of X' stays inside the bound
    want_exact = oracle.gemm(packing, ref_packed, li.scales, xr_exact, k)
    assert oracle.rel_err(y, want_exact) < TOL


def test_gemm_base3_equals_2bit():
    note("gemm base-3 and 2-bit of the same trits agree exactly")
    g = synth.rng(231, 0, 0, 0)
    m, n, k = 130, 300, 1280      # M > 96: the tiled prefill kernel
    t = synth.trits(g, n, k)
    s = scales_dev(synth.scales_f16(g, n, k))
    xr = dev(g.standard_normal((m, k)).astype(np.float16))
    p2, p3 = dev(oracle.pack_2bit(t)[0]), dev(oracle.pack_base3(t)[0])
    y2 = host(tb.tb_gemm("2bit", p2, s, xr))
    y3 = host(tb.tb_gemm("base3", p3, s, xr))
    assert np.array_equal(y2, y3)
    # a few rows run on the batched decode kernel: the same holds there
    y2 = host(tb.tb_gemm("2bit", p2, s, xr[:20].contiguous()))
    y3 = host(tb.tb_gemm("base3", p3, s, xr[:20].contiguous()))
    assert np.array_equal(y2, y3)


# ------------------------------------------------------------------ measurement aid

@pytest.mark.parametrize("nbytes", [16, 4096, 32768 + 48, 19496960, 300 << 20])
def test_stream_read_touches_every_word_once(nbytes):
    """The read-ceiling kernel reads each 32-bit word exactly once: the XOR of its
    per-workgroup words equals the XOR of the buffer (every word distinct here)."""
    note(f"stream read {nbytes} bytes")
    words = nbytes // 4
    g = synth.rng(270, 0, nbytes % 251, 0)
    host_buf = g.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = dev(host_buf.view(np.int32))
    sink = torch.zeros(tb.TB_STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    tb.tb_stream_read(buf, sink)
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(host_buf)
