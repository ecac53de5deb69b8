"""Compile the plain C++ oracle (oracle/cpp/ternary_oracle.cpp) into a host shared library.

Test infrastructure only, like the rest of ``oracle``: the tests and the
benchmark's CPU-baseline leg load it; the HIP library never does.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "ternary_oracle.cpp")
LIB = os.path.join(HERE, "cpp", "libternary_oracle.so")


def build() -> str:
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        raise RuntimeError("no host C++ compiler (g++) found for the C++ oracle")
    tmp = LIB + ".tmp"
    cmd = [cxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", tmp]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{proc.stdout}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
