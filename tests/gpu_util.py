"""Helpers for the GPU parity tests (not collected): host arrays <-> device tensors."""
import sys

import numpy as np
import torch

import synth

DEV = "cuda"
TOL = 2e-3          # max relative error bound on products (row-rms floored)


def note(msg):
    """Name the case on stderr before the GPU step runs."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def signs_dev(bits):
    return dev(np.asarray(bits, dtype=np.uint32).view(np.int32))


def scales_dev(bits):
    return dev(np.asarray(bits, dtype=np.uint16).view(np.float16))


def act_dev(x, x_dtype):
    if x_dtype == "bf16":
        return dev(np.asarray(x, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return dev(np.asarray(x, dtype=np.float32))


def act_f64(x, x_dtype):
    return synth.bf16_bits_to_f64(x) if x_dtype == "bf16" else np.asarray(x, dtype=np.float64)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def f16_ulp_distance(a, b):
    """Distance in fp16 units in the last place between two fp16 arrays (same sign assumed near 0)."""
    ia = np.asarray(a, dtype=np.float16).view(np.int16).astype(np.int64)
    ib = np.asarray(b, dtype=np.float16).view(np.int16).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)
