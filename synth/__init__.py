"""Seeded synthetic inputs for the ternary rotated-basis linear.

This module only draws inputs: ternary weights, group scales, activations and
the sign diagonal.  It holds none of the method's arithmetic (no packing, no
rotation, no products), so both the reference oracle and the HIP path can take
their inputs from here without sharing any compute code.

Every draw comes from numpy's Philox4x32-10 counter-based generator keyed by a
(workload, tensor) pair, so a tensor is reproducible on its own, whatever else
was drawn before it.

Distributions (the workloads the pages measure are whole ternary models; these
stand-in shapes and statistics are synthetic):
  * trits: two generator bits per weight, 00 -> -1, 11 -> +1, 01/10 -> 0, so
    P(0) = 1/2 and P(+1) = P(-1) = 1/4 exactly;
  * group scales: |N(0, 0.02)| + 1e-3, rounded once to fp16 (round to nearest
    even), one per 128 consecutive weights of a row;
  * activations: N(0, 1) in fp64, optionally with round(0.001 K) outlier
    channels (the same channels in every row) multiplied by 20, then rounded
    to float32 and, for bf16 inputs, to bf16 (round to nearest even);
  * sign diagonal: 1024 fair bits (set = -1), tiled over every 1024-block of K;
  * full-precision weights (for the ternariser): N(0, 0.02^2), optionally with
    outlier input columns multiplied by 20, rounded once to float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

GROUP = 128        # weights per fp16 scale
BLOCK = 1024       # rotation block size n
KEY_BASE = 0x7B500000

# tensor ids inside a workload key
T_TRITS, T_SCALES, T_X, T_SIGNS, T_OUTLIERS, T_FP_WEIGHTS = 0, 1, 2, 3, 4, 5


def rng(workload: int, tensor: int, layer: int = 0, linear: int = 0) -> np.random.Generator:
    """Independent Philox stream for one tensor of one workload."""
    key = ((KEY_BASE + workload) << 32) | (tensor << 24) | (layer << 8) | linear
    return np.random.Generator(np.random.Philox(key=key))


def trits(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 [n][k] ternary weights, P(0)=1/2, P(+-1)=1/4, from two bits each."""
    r = g.integers(0, 4, size=(n, k), dtype=np.uint8)
    t = np.zeros((n, k), dtype=np.int8)
    t[r == 0] = -1
    t[r == 3] = 1
    return t


def scales_f16(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    """uint16 [n][k/128]: fp16 bit patterns of |N(0, 0.02)| + 1e-3."""
    if k % GROUP:
        raise ValueError("k must be a multiple of 128")
    s = np.abs(g.standard_normal((n, k // GROUP))) * 0.02 + 1e-3
    return s.astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact value of fp16 bit patterns."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def outlier_channels(g: np.random.Generator, k: int, frac: float = 0.001) -> np.ndarray:
    count = int(round(frac * k))
    return np.sort(g.choice(k, size=count, replace=False)) if count else np.zeros(0, np.int64)


def activations(g: np.random.Generator, rows: int, k: int, outliers: np.ndarray | None = None,
                dtype: str = "bf16") -> np.ndarray:
    """[rows][k] activations: uint16 bf16 bits (dtype='bf16') or float32."""
    x = g.standard_normal((rows, k))
    if outliers is not None and len(outliers):
        x[:, outliers] *= 20.0
    x32 = x.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return x32
    raise ValueError(dtype)


def fp_weights(g: np.random.Generator, n: int, k: int, std: float = 0.02,
               outliers: np.ndarray | None = None, gain: float = 20.0) -> np.ndarray:
    """float32 [n][k] full-precision weights (y = W x): N(0, std^2), with the given
    input columns multiplied by ``gain`` before the single rounding to float32."""
    w = g.standard_normal((n, k)) * std
    if outliers is not None and len(outliers):
        w[:, outliers] *= gain
    return w.astype(np.float32)


def sign_bits(g: np.random.Generator, k: int) -> np.ndarray:
    """uint32 [k/32]: bit b of word w is channel 32w+b; set means -1.

    One 1024-entry diagonal is drawn and repeated over every block of k.
    """
    if k % BLOCK:
        raise ValueError("k must be a multiple of 1024")
    bits = g.integers(0, 2, size=BLOCK, dtype=np.uint64)
    words = (bits.reshape(BLOCK // 32, 32) << np.arange(32, dtype=np.uint64)).sum(
        axis=1, dtype=np.uint64).astype(np.uint32)
    return np.tile(words, k // BLOCK)


@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    n: int  # output rows
    k: int  # input features


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    linears: tuple
    batches: tuple
    packings: tuple
    x_dtype: str
    outliers: bool
    description: str


HIDDEN, FFN = 5120, 17408

BLOCK_LINEARS = (
    Linear("q", HIDDEN, HIDDEN), Linear("k", HIDDEN, HIDDEN), Linear("v", HIDDEN, HIDDEN),
    Linear("o", HIDDEN, HIDDEN), Linear("gate", FFN, HIDDEN), Linear("up", FFN, HIDDEN),
    Linear("down", HIDDEN, FFN),
)

WORKLOADS = {
    0: Workload(0, "linear1024_2bit_b1", (Linear("w", 1024, 1024),), (1,), ("2bit",), "f32", False,
                "single 1024x1024 ternary linear, 2-bit codes, batch 1, fp32 activations"),
    1: Workload(1, "gemv_ffn_17408x5120_base3_b1", (Linear("gate", FFN, HIDDEN),), (1,), ("base3",),
                "bf16", True,
                "decode GEMV N=17408 K=5120 batch 1, base-3 codes, bf16 activations with 0.1% x20 outliers"),
    2: Workload(2, "block_linears_b1_b8", BLOCK_LINEARS, (1, 8), ("2bit", "base3"), "bf16", False,
                "one block's q/k/v/o, gate/up, down linears at batch 1 and 8, both packings"),
    3: Workload(3, "pp512_gemm_17408x5120_2bit", (Linear("gate", FFN, HIDDEN),), (512,), ("2bit",),
                "bf16", True,
                "prefill GEMM M=512 N=17408 K=5120, 2-bit codes, bf16 activations with outliers"),
    4: Workload(4, "decode_stream_64layers_base3", BLOCK_LINEARS, (1,), ("base3",), "bf16", False,
                "64 layers x block linears, base-3, batch 1 (one decode token's weight stream)"),
}


@dataclasses.dataclass
class LinearInputs:
    trits: np.ndarray      # int8 [n][k]
    scales: np.ndarray     # uint16 fp16 bits [n][k/128]
    x: np.ndarray          # uint16 bf16 bits or float32, [rows][k]
    x_dtype: str
    signs: np.ndarray      # uint32 [k/32]
    outliers: np.ndarray


def linear_inputs(wid: int, n: int, k: int, rows: int, x_dtype: str, outliers: bool,
                  layer: int = 0, linear: int = 0) -> LinearInputs:
    """All seeded inputs of one linear of a workload."""
    t = trits(rng(wid, T_TRITS, layer, linear), n, k)
    s = scales_f16(rng(wid, T_SCALES, layer, linear), n, k)
    oc = outlier_channels(rng(wid, T_OUTLIERS, layer, linear), k) if outliers else np.zeros(0, np.int64)
    x = activations(rng(wid, T_X, layer, linear), rows, k, oc, x_dtype)
    sg = sign_bits(rng(wid, T_SIGNS), k)
    return LinearInputs(t, s, x, x_dtype, sg, oc)
