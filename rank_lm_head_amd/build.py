"""Builds liblrhead.so (and the benchmark's read probe, libprobe.so) in-tree
with hipcc for gfx950.

    python -m rank_lm_head_amd.build

Cross-compiles without a GPU. Each source becomes an object of its own, the
objects are compiled in parallel and then linked into the shared library.
Packed fp32 instructions are disabled for the device code; hipcc's host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblrhead.so")
PROBE_LIB = os.path.join(PKG, "libprobe.so")   # measurement only, not the head's ABI
PROBE_SOURCE = "probe_read.hip"
OBJ = os.path.join(PKG, "_build")
SOURCES = ["kernels_small.hip", "kernels_mfma.hip", "kernels_gemm.hip", "kernels_merge.hip", "kernels_branch.hip",
           "kernels_factor.hip", "kernels_b1.hip", "lrhead.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Werror=return-type", "-Werror=infinite-recursion",
]
NOISE = "is not a recognized feature for this target"


def _run(cmd: list[str]) -> tuple[int, list[str]]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [HIPCC, *FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", obj]))
    probe_tmp = PROBE_LIB + ".tmp"
    probe = [HIPCC, *FLAGS, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_tmp]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        probe_job = ex.submit(_run, probe)
        results = list(ex.map(lambda j: _run(j[1]), jobs))
        probe_res = probe_job.result()
    if probe_res[0] != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(probe) + "\n" + "\n".join(probe_res[1]))
    os.replace(probe_tmp, PROBE_LIB)
    out = []
    for (obj, cmd), (rc, msgs) in zip(jobs, results):
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
        out += msgs
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
    rc, msgs = _run(link)
    if rc != 0:
        raise RuntimeError("link failed:\n" + " ".join(link) + "\n" + "\n".join(msgs))
    out += msgs
    if verbose and out:
        print("\n".join(out), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
