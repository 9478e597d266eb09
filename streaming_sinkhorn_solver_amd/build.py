"""Build the HIP library ``libfs_sinkhorn.so`` in-tree for gfx950.

Every translation unit under ``csrc/`` is compiled with hipcc for
``--offload-arch=gfx950`` (packed fp32 instructions disabled) and linked into
one shared library next to this file, which the ctypes binding loads.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfs_sinkhorn.so")
SOURCES = ["fs_api.cpp", "fs_prep.hip", "fs_lse.hip", "fs_lse_small.hip", "fs_transport.hip",
           "fs_grad.hip", "fs_probe.hip", "fs_hvp.hip", "fs_bsparse.hip", "fs_static.hip",
           "fs_persistent.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    rest = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    if rest:
        print(f"[build] {src}:\n{rest}", file=sys.stderr)


def build(verbose: bool = True, out: str = LIB) -> str:
    """Compile all sources (always) and link the library; returns its path."""
    tmp = tempfile.mkdtemp(prefix="fs_build_")
    try:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1]), zip(SOURCES, objs)))
        out_tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + objs
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        os.replace(out_tmp, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    if verbose:
        print(f"[build] {out}")
    return out


if __name__ == "__main__":
    build()
