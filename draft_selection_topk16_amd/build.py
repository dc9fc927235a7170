"""Build libdflash2.so (HIP, gfx950) in-tree with hipcc.

    python -m draft_selection_topk16_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "dflash2.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdflash2.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"),
        # never emit packed fp32 arithmetic
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False) -> str:
    """Compile the HIP library; always recompiles."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags() + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libdflash2.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
