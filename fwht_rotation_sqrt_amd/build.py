"""Compile the HIP sources of the package into libtb.so for gfx950 (in-tree).

Each .hip file is compiled to an object in parallel, then linked into one
shared library next to this file.  The library is replaced atomically, so a
concurrent loader sees either the old or the new file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtb.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the generated code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-function"]
# Per-file device flags.  The prefill product keeps 136 accumulators per lane
# live across its K loop; in the accumulation-register form the compiler
# copies them between registers around every matrix instruction, in the
# VGPR form it updates them in place.
FILE_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              # the batch-1 decode kernel's arguments arrive in SGPRs at wave launch instead of
              # through a scalar load of the argument segment, which waits behind the weight stream
              "decode1.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtb.so)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{proc.stdout}")
    return proc.stdout


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objects = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in sources]

    def compile_one(pair):
        src, obj = pair
        extra = FILE_FLAGS.get(os.path.basename(src), [])
        return _run([hipcc, *COMMON, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj])

    jobs = jobs or min(len(sources), os.cpu_count() or 4, 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        for out in pool.map(compile_one, zip(sources, objects)):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objects, "-o", tmp])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
