"""Build libuhla.so (HIP, gfx950) in-tree with hipcc.

    python -m global_attention_image_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libuhla.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        # packed fp32 VALU ops stay disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


def build(verbose: bool = True) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
