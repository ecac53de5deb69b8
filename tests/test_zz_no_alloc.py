"""The entry point that allocates nothing (tb_linear_noalloc) against the one with a caller
workspace (tb_linear_ws), through the C ABI, on two calls in a row, the second smaller."""
import ctypes

import numpy as np
import pytest
import torch

import fwht_rotation_sqrt_amd as tb
import oracle
import synth
from gpu_util import TOL, dev, host, note, scales_dev, signs_dev

pytestmark = pytest.mark.gpu


def _case(packing, n, k, rows, seed):
    g = synth.rng(290, seed, n % 251, k // 1024)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x = g.standard_normal((rows, k)).astype(np.float32)
    packed, _ = (oracle.pack_2bit if packing == "2bit" else oracle.pack_base3)(t)
    want = oracle.gemv(packing, packed, s, oracle.rotate(x.astype(np.float64), signs), k)
    return dev(packed), scales_dev(s), dev(x), signs_dev(signs), want


def _noalloc(packing, pd, sd, xd, sgn, y):
    lib = tb.library()
    b, k = xd.shape
    n = pd.shape[0]
    st = lib.tb_linear_noalloc(tb.PACKINGS[packing], ctypes.c_void_p(pd.data_ptr()), ctypes.c_void_p(sd.data_ptr()),
                               ctypes.c_void_p(xd.data_ptr()), tb.TB_F32, ctypes.c_void_p(sgn.data_ptr()),
                               ctypes.c_void_p(y.data_ptr()), b, n, k,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, tb.TBError("tb_linear_noalloc", st)


@pytest.mark.parametrize("packing", ["2bit", "base3"])
def test_noalloc_matches_workspace_entry_point(packing):
    # call 1: 32 rows of K = 17408 (2.2 MB of the 4 MiB scratch); call 2: 9 rows of K = 3072;
    # call 3: 6 rows of K = 5120 (x' rotated into the array, then the limb product)
    for (n, k, rows), seed in (((300, 17408, 32), 0), ((200, 3072, 9), 1), ((500, 5120, 6), 2)):
        note(f"noalloc {packing} n={n} k={k} rows={rows}")
        pd, sd, xd, sgn, want = _case(packing, n, k, rows, seed)
        assert tb.tb_linear_workspace_bytes(packing, rows, n, k) > 0   # the call uses the scratch
        y0 = torch.full((rows, n), float("nan"), dtype=torch.float32, device="cuda")
        _noalloc(packing, pd, sd, xd, sgn, y0)
        y1 = tb.tb_linear_ws(packing, pd, sd, xd, sgn)
        a, b = host(y0), host(y1)
        assert np.array_equal(a, b)                                     # same kernels, same x'
        assert oracle.rel_err(a, want) < TOL


def test_noalloc_batch1_rows_in_parts():
    """Batch 1, base-3, K = 17408: the partial sums of the row's four parts of K go to the static
    array; then a smaller split call (K = 6144, two parts) on the same array.  Same bits as the
    workspace entry point."""
    for (n, k), seed in (((700, 17408), 3), ((300, 6144), 4)):
        note(f"noalloc base3 batch 1 n={n} k={k}")
        pd, sd, xd, sgn, want = _case("base3", n, k, 1, seed)
        assert tb.tb_linear_workspace_bytes("base3", 1, n, k) > 0
        y0 = torch.full((1, n), float("nan"), dtype=torch.float32, device="cuda")
        _noalloc("base3", pd, sd, xd, sgn, y0)
        a, b = host(y0), host(tb.tb_linear_ws("base3", pd, sd, xd, sgn))
        assert np.array_equal(a, b)
        assert oracle.rel_err(a, want) < TOL


def test_noalloc_small_batches_and_limit():
    pd, sd, xd, sgn, want = _case("base3", 64, 2048, 4, 2)
    y = torch.empty((4, 64), dtype=torch.float32, device="cuda")
    _noalloc("base3", pd, sd, xd, sgn, y)                              # the fused kernel, no scratch
    assert oracle.rel_err(host(y), want) < TOL
    lib = tb.library()
    assert lib.tb_linear_noalloc(1, 16, 16, 16, 0, 16, 16, 32, 8, 1 << 16, None) == 8  # beyond 4 MiB


def test_noalloc_batched_without_room_for_parts():
    """32 rows of K = 17408 on 2048 weight rows: x' (2.2 MB) and the partial sums of the batched
    product's eight parts of K (2.1 MB) together pass the 4 MiB array, so the call takes whole
    rows (x' only).  Against the oracle on sampled rows, and within the tolerance of the
    workspace entry point, which takes the parts (another summation order)."""
    n, k, rows = 2048, 17408, 32
    assert tb.tb_linear_workspace_bytes("base3", rows, n, k) > (4 << 20) >= 4 * rows * k
    note(f"noalloc base3 n={n} k={k} rows={rows} without parts")
    g = synth.rng(290, 7, n % 251, k // 1024)
    t = synth.trits(g, n, k)
    s = synth.scales_f16(g, n, k)
    signs = synth.sign_bits(g, k)
    x = g.standard_normal((rows, k)).astype(np.float32)
    packed, _ = oracle.pack_base3(t)
    sample = np.unique(np.concatenate([np.arange(0, n, 17), [n - 1]]))
    want = oracle.gemv("base3", packed[sample], s[sample], oracle.rotate(x.astype(np.float64), signs), k)
    pd, sd, xd, sgn = dev(packed), scales_dev(s), dev(x), signs_dev(signs)
    y0 = torch.full((rows, n), float("nan"), dtype=torch.float32, device="cuda")
    _noalloc("base3", pd, sd, xd, sgn, y0)
    a = host(y0)
    assert oracle.rel_err(a[:, sample], want) < TOL
    assert oracle.rel_err(a, host(tb.tb_linear_ws("base3", pd, sd, xd, sgn))) < TOL
