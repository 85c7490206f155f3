"""Builds liblrhead.so in-tree with hipcc for gfx950.

    python -m rank_lm_head_amd.build

Cross-compiles without a GPU. Packed fp32 instructions are disabled for the
device code; hipcc's host pass warns that it does not know that feature,
which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblrhead.so")
SOURCES = ["kernels_small.hip", "kernels_mfma.hip", "kernels_gemm.hip", "kernels_merge.hip", "kernels_branch.hip",
           "kernels_factor.hip", "lrhead.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Werror=return-type", "-Werror=infinite-recursion",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
