"""Build the CPU oracle (liboracle.so) from its C++17 sources with g++.

Test infrastructure only. Flags: -O2 with IEEE arithmetic kept intact
(-fno-fast-math, -ffp-contract=off: no fused multiply-add, no reassociation),
OpenMP across independent units only.

Usage: python oracle/build.py
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["quant.cpp", "attention.cpp", "sage.cpp"]
LIB = os.path.join(HERE, "liboracle.so")
CXX = os.environ.get("ORACLE_CXX", "g++")
FLAGS = ["-O2", "-std=c++17", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall",
         "-Wextra", "-Wno-unused-parameter"]


def build(src_dir: str = HERE, out: str = LIB) -> str:
    """Compile the oracle sources found in src_dir into the shared library
    `out` (always rebuilds). Returns its path."""
    tmp = out + ".tmp"
    cmd = [CXX, *FLAGS, f"-I{src_dir}", *[os.path.join(src_dir, s) for s in SOURCES], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
