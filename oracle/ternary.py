"""Reference oracle for y = W(Rx) on packed ternary weights (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg use
this module.  It is a plain float64 numpy transcription of what the pages
define, shares nothing with the HIP path, and is deliberately slow.

Pages cited (title, address, section):
  [P1] "Bonsai low-bit learning path" (adenzhou1350.github.io/learn/bonsai-low-bit/),
       section "Understand 1.6 bit with five numbers": five trits t_i in {-1,0,1}
       are stored in one byte as sum_i (t_i + 1) * 3**i, since 3**5 = 243 <= 256,
       and recovered as (byte // 3**i) % 3 - 1.
  [P4] "TensorSharp view of Ternary Bonsai 2 27B" (2kiu.com/news/5337570/):
       section 1.2 (bits per weight = stored bytes * 8 / parameters),
       section 2.1 (blockwise ternarisation: each block has its own scale, taken
       from the mean absolute weight times a correction; w/scale >= thr -> +1,
       <= -thr -> -1, otherwise 0; the finer form tries a set of candidate
       thresholds and keeps the one with the least reconstruction error),
       section 3.1 (H is a +-1 matrix with H H^T = n I),
       section 3.2 (Sylvester construction, printed H_4),
       section 5.2 (butterfly fast Hadamard divided by sqrt(n)).
  [P5] "Ternary Bonsai 2 27B release" (linlog.top/article/1481), section
       "How the ternary weights reach 1.76 bit": ternary weights with one fp16
       scale per 128 weights (g128); the fixed rotated basis
       R = (1/sqrt(n)) H_n S with n = 1024 and S a fixed +-1 diagonal, applied
       blockwise, and inference computes f(x) = W(Rx); the weights are moved into
       that basis before they are ternarised.

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):
  * 2-bit code: c = t + 1 (00 -> -1, 01 -> 0, 10 -> +1, 11 invalid); weight k
    of a row sits in bits 2(k mod 4)..2(k mod 4)+1 of byte k // 4, i.e. a row is
    the little-endian base-4 number sum_k c_k 4**k (the base-4 twin of [P1]).
  * base-3 layout: every group of 128 weights takes 26 bytes; bytes 0..24 hold
    weights 5j..5j+4 by the [P1] formula (first trit least significant); byte 25
    holds weights 125..127 and two pad trits equal to 0 (digit 1), so the last
    byte of a group lies in 108..134.  1.75 bits per weight before scales.
  * scales: fp16 [N][K/128] row-major, groups are consecutive 128-slices of K.
  * H ordering: Sylvester (natural) order, H[i][j] = (-1)**popcount(i & j),
    which is the recursion of [P4] section 3.2.
  * R: S first, then H, then 1/sqrt(1024) = 1/32; blocks are consecutive
    1024-slices of K; the sign diagonal is a K-bit mask (bit set = -1).
  * weights into the basis: W' = W R_K^T, so that W x = W' (R_K x) exactly;
    each row w of W becomes R_K w, the same transform as an activation row.
  * ternariser, per 128-group of W' (the scale groups): with a = mean |w|, the
    candidate thresholds are c_j a, c_j = (j + 1) / 32 for j = 0..63; candidate
    j keeps the weights with |w| >= c_j a as sign(w) and zeroes the rest; its
    scale is the least-squares scale of those trits (the mean kept magnitude,
    i.e. a times a correction factor) rounded to fp16 (nearest even); its error
    is the group's squared reconstruction error with that rounded scale
    (infinite when the scale overflows fp16).  The least error wins, the
    lowest j on ties.  An all-zero group gives zero trits
    and scale 0; a group holding a non-finite value, or whose chosen scale
    overflows fp16, is counted bad and stored as zero trits with scale 0.
    Every step runs in float64.
"""
from __future__ import annotations

import numpy as np

GROUP = 128                 # weights per fp16 scale  [P5]
BLOCK = 1024                # rotation block size n   [P5]
B3_TRITS_PER_BYTE = 5       # [P1]
B3_BYTES_PER_GROUP = 26     # ceil(128 / 5): 125 trits in 25 bytes + 3 trits and 2 pads
POW3 = np.array([1, 3, 9, 27, 81], dtype=np.int64)


def _check_trits(trits: np.ndarray) -> tuple[np.ndarray, int]:
    """Invalid trits (not in {-1,0,1}) are counted and stored as 0."""
    t = np.asarray(trits).astype(np.int64)
    bad = (t < -1) | (t > 1)
    return np.where(bad, 0, t), int(bad.sum())


# ---------------------------------------------------------------- packing

def pack_2bit(trits: np.ndarray) -> tuple[np.ndarray, int]:
    """int8 [N][K] -> uint8 [N][K/4]: byte j = sum_{i<4} (t_{4j+i} + 1) << 2i."""
    t, bad = _check_trits(trits)
    n, k = t.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    c = (t + 1).reshape(n, k // 4, 4)
    packed = (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)
    return packed, bad


def unpack_2bit(packed: np.ndarray, k: int) -> tuple[np.ndarray, int]:
    """uint8 [N][K/4] -> int8 [N][K]; code 11 is invalid: counted, decoded as 0."""
    p = np.asarray(packed, dtype=np.int64)
    n = p.shape[0]
    codes = np.stack([(p >> (2 * i)) & 3 for i in range(4)], axis=-1).reshape(n, k)
    bad = codes == 3
    t = np.where(bad, 0, codes - 1).astype(np.int8)
    return t, int(bad.sum())


def pack_base3(trits: np.ndarray) -> tuple[np.ndarray, int]:
    """int8 [N][K] -> uint8 [N][26*K/128] by the [P1] formula, per 128-group.

    Each group of 128 trits is extended by two 0 trits to 130 = 26 * 5, and each
    consecutive run of five becomes one byte sum_i (t_i + 1) * 3**i.
    """
    t, bad = _check_trits(trits)
    n, k = t.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = t.reshape(n, k // GROUP, GROUP)
    g = np.concatenate([g, np.zeros((n, k // GROUP, 2), dtype=np.int64)], axis=2)
    digits = (g + 1).reshape(n, k // GROUP, B3_BYTES_PER_GROUP, B3_TRITS_PER_BYTE)
    packed = (digits * POW3).sum(axis=-1)
    return packed.reshape(n, -1).astype(np.uint8), bad


def unpack_base3(packed: np.ndarray, k: int) -> tuple[np.ndarray, int]:
    """uint8 [N][26*K/128] -> int8 [N][K] by (byte // 3**i) % 3 - 1  [P1].

    A byte >= 243 is not a base-3 code: it counts once and its trits decode as
    0.  A valid last byte of a group whose two pad digits are not 1 (pad trit
    0) counts once; its three real trits still decode by the formula.
    """
    p = np.asarray(packed, dtype=np.int64)
    n = p.shape[0]
    groups = k // GROUP
    p = p.reshape(n, groups, B3_BYTES_PER_GROUP)
    over = p >= 243
    digits = (p[..., None] // POW3) % 3                      # [n][g][26][5]
    t = np.where(over[..., None], 0, digits - 1)
    pad_digits = digits[..., B3_BYTES_PER_GROUP - 1, 3:]
    bad_pad = (~over[..., B3_BYTES_PER_GROUP - 1]) & np.any(pad_digits != 1, axis=-1)
    t = t.reshape(n, groups, B3_BYTES_PER_GROUP * B3_TRITS_PER_BYTE)[..., :GROUP]
    return t.reshape(n, k).astype(np.int8), int(over.sum() + bad_pad.sum())


def packed_row_bytes(packing: str, k: int) -> int:
    if k % GROUP:
        return -1
    return k // 4 if packing == "2bit" else B3_BYTES_PER_GROUP * (k // GROUP)


def bits_per_weight(packing: str, k: int, with_scales: bool = True) -> float:
    """Stored bytes * 8 / parameters for one row  [P4 section 1.2]."""
    nbytes = packed_row_bytes(packing, k) + (2 * (k // GROUP) if with_scales else 0)
    return nbytes * 8 / k


# ---------------------------------------------------------------- rotation

def hadamard(n: int) -> np.ndarray:
    """Sylvester-ordered Walsh-Hadamard matrix, H[i][j] = (-1)**popcount(i & j)."""
    if n & (n - 1):
        raise ValueError("n must be a power of two")
    i = np.arange(n, dtype=np.int64)
    ij = i[:, None] & i[None, :]
    pop = np.zeros_like(ij)
    while ij.any():
        pop += ij & 1
        ij >>= 1
    return np.where(pop & 1, -1.0, 1.0)


def sign_vector(sign_bits: np.ndarray, k: int) -> np.ndarray:
    """K-bit mask (bit b of word w is channel 32w+b; set = -1) -> +-1 float64 [K]."""
    w = np.asarray(sign_bits, dtype=np.uint64)
    ch = np.arange(k)
    bit = (w[ch // 32] >> (ch % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(bit == 1, -1.0, 1.0)


def rotate(x: np.ndarray, sign_bits: np.ndarray) -> np.ndarray:
    """x' = R_K x with R_K = blockdiag(H_1024 S_beta / 32)  [P5], explicit product.

    x: float64 [rows][K], K a multiple of 1024.  Each 1024-block beta of each
    row becomes H (S_beta * x_beta) / 32; H is symmetric, so x_beta' = (S x_beta) H / 32.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 1024")
    h = hadamard(BLOCK)
    xs = (x * sign_vector(sign_bits, k)).reshape(rows, k // BLOCK, BLOCK)
    return (xs @ h.T / np.sqrt(BLOCK)).reshape(rows, k)


# ---------------------------------------------------------------- products

def dequantize(packing: str, packed: np.ndarray, scales_bits: np.ndarray, k: int) -> np.ndarray:
    """W_hat[n][k] = s[n][k // 128] * t[n][k] in float64; trits decoded from the bytes."""
    t, _ = unpack_2bit(packed, k) if packing == "2bit" else unpack_base3(packed, k)
    s = np.asarray(scales_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return t.astype(np.float64) * np.repeat(s, GROUP, axis=1)


def gemv(packing: str, packed: np.ndarray, scales_bits: np.ndarray, xr: np.ndarray, k: int) -> np.ndarray:
    """y[b][n] = sum_gamma s[n][gamma] sum_{k in gamma} t[n][k] xr[b][k]  (float64).

    xr are the rotated activations exactly as handed to the product.
    """
    w = dequantize(packing, packed, scales_bits, k)
    return np.asarray(xr, dtype=np.float64) @ w.T


def gemm(packing: str, packed: np.ndarray, scales_bits: np.ndarray, xr: np.ndarray, k: int) -> np.ndarray:
    """Prefill product Y[m][n] = sum_k X'[m][k] W_hat[n][k]; same definition as gemv."""
    return gemv(packing, packed, scales_bits, xr, k)


# ---------------------------------------------------------------- ternariser

TERNARY_CANDIDATES = 64     # thresholds (j + 1) / 32 * mean|w|, j = 0..63


def rotate_weights(w: np.ndarray, sign_bits: np.ndarray) -> np.ndarray:
    """W' = W R_K^T in float64, so that W x = W' (R_K x)  [P5].

    Row n of W' is R_K applied to row n of W, i.e. ``rotate`` on the rows.
    """
    return rotate(np.asarray(w, dtype=np.float64), sign_bits)


def f64_to_f16_bits(v) -> np.ndarray:
    """float64 -> nearest fp16 (ties to even), one rounding; uint16 bit patterns."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def ternarize(wr: np.ndarray):
    """Rotated weights [N][K] -> (int8 trits [N][K], uint16 fp16 scale bits [N][K/128],
    chosen candidate [N][K/128] (-1 for zero or bad groups), bad group count)  [P4 section 2.1].

    Each 128-group is searched over the candidate thresholds independently; see
    the module notes for the reading of the scale, threshold and error.
    """
    wr = np.asarray(wr, dtype=np.float64)
    n, k = wr.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    with np.errstate(over="ignore", invalid="ignore"):
        return _ternarize_groups(wr, n, k)


def _ternarize_groups(wr, n, k):
    g = wr.reshape(n * (k // GROUP), GROUP)
    mag = np.abs(g)
    finite = np.all(np.isfinite(g), axis=1)
    a = np.sum(np.where(finite[:, None], mag, 0.0), axis=1) / GROUP       # mean |w|
    best_err = np.full(len(g), np.inf)
    best_j = np.zeros(len(g), dtype=np.int64)
    best_s16 = np.zeros(len(g), dtype=np.uint16)
    for j in range(TERNARY_CANDIDATES):
        theta = (j + 1) / 32 * a
        keep = mag >= theta[:, None]
        nnz = np.sum(keep, axis=1)
        kept_sum = np.sum(np.where(keep, mag, 0.0), axis=1)
        s = np.divide(kept_sum, nnz, out=np.zeros(len(g)), where=nnz > 0)
        s16_bits = f64_to_f16_bits(s)
        s16 = s16_bits.view(np.float16).astype(np.float64)
        err = np.sum(np.where(keep, (mag - s16[:, None]) ** 2, mag * mag), axis=1)
        better = (err < best_err) | (j == 0)
        best_err = np.where(better, err, best_err)
        best_j = np.where(better, j, best_j)
        best_s16 = np.where(better, s16_bits, best_s16)
    theta = (best_j + 1) / 32 * a
    trits = np.where(mag >= theta[:, None], np.sign(g), 0.0).astype(np.int8)
    bad = ~finite | ~np.isfinite(best_s16.view(np.float16))
    zero = (a == 0) | bad
    trits[zero] = 0
    best_s16 = np.where(zero, 0, best_s16).astype(np.uint16)
    best_j = np.where(zero, -1, best_j)
    return (trits.reshape(n, k), best_s16.reshape(n, k // GROUP), best_j.reshape(n, k // GROUP),
            int(np.sum(bad)))


def quantize_weights(w: np.ndarray, sign_bits: np.ndarray):
    """fp weights W [N][K] (y = W x) -> ternarize(W R_K^T): the offline step that
    puts W into the rotated basis and onto the g128 ternary grid  [P5], [P4 section 2.1]."""
    return ternarize(rotate_weights(w, sign_bits))


# ---------------------------------------------------------------- error metric

def rel_err(y: np.ndarray, yref: np.ndarray) -> float:
    """max_i |y_i - yref_i| / max(|yref_i|, rms(yref row)), rows = leading dims.

    A bare |yref_i| denominator is ill-posed for outputs that cancel to near
    zero; the row rms floor keeps the bound meaningful for them.
    """
    y = np.asarray(y, dtype=np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    yr = yref.reshape(-1, yref.shape[-1])
    rms = np.sqrt(np.mean(yr * yr, axis=1, keepdims=True))
    den = np.maximum(np.abs(yr), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y.reshape(yr.shape) - yr) / den)) if yr.size else 0.0


def normwise_err(y: np.ndarray, yref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    d = np.linalg.norm(yref)
    return float(np.linalg.norm(y - yref) / d) if d else float(np.linalg.norm(y))
