"""Compile the CPU oracle (``oracle.c``) into ``liboracle.so`` with gcc.

Test infrastructure: run by ``__graft_entry__.build()`` and on first use by
the oracle wrapper.  Portable x86-64 code (no -march=native, since the library
may run on another host than the one that built it), IEEE arithmetic (no
-ffast-math), OpenMP for the output-index loops.
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
OUT = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(OUT) and os.path.getmtime(OUT) >= os.path.getmtime(SRC):
        return OUT
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(force=True))
    sys.exit(0)
