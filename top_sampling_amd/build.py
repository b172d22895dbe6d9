"""Build ``libtopsampling.so`` (gfx950 only) in-tree with hipcc.

Usage: ``python top_sampling_amd/build.py`` (or ``build()`` after loading this
file by path; importing the package loads the library, so this script never
imports it).  Every call recompiles every source.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtopsampling.so")
SOURCES = ["api.hip", "lmhead_gemm.hip", "lmhead_fp8.hip", "sampler_fast.hip", "sampler_exact.hip",
           "assemble.hip", "clock_probe.hip", "noise_readout.hip", "noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 instructions stay off in every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd: list[str]) -> str:
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
