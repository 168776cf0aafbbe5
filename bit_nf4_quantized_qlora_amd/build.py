"""Build libqlora.so (gfx950) in-tree from csrc/*.hip with hipcc.

Every call recompiles: the objects go to ``_build/`` next to this file and the
shared library to ``libqlora.so`` beside them.  A second library from the
same sources, ``libqlora_prof.so``, is built with -DQLORA_PROFILE: it adds
the per-kernel event timer (profile.hip, include/qlora_profile.h) that the
benchmark's tracing pass uses, and the matrix-core peak microbenchmark
(peak.hip); the product library carries neither.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqlora.so")
LIB_PROF = os.path.join(PKG, "libqlora_prof.so")
SOURCES = ["capi.hip", "quantize.hip", "dequant.hip", "lora_gemm.hip", "jobs.hip", "nf4_tile.hip", "nf4_gemv.hip", "linear_fwd.hip", "linear_bwd.hip", "merge.hip", "adamw.hip", "swiglu.hip", "attention.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # every multiply and add is rounded on its own (the block scale is defined
    # with two roundings); HIP would otherwise contract a*b+c into an FMA
    "-ffp-contract=off",
    # packed fp32 VALU ops stay off: the kernels use scalar fp32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in p.stderr.splitlines() if "not a recognized feature" not in ln)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(jobs: int | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    variants = [(LIB, os.path.join(BUILD, "lib"), SOURCES, []),
                (LIB_PROF, os.path.join(BUILD, "prof"), SOURCES + ["profile.hip", "peak.hip"], ["-DQLORA_PROFILE=1"])]
    cmds, links = [], []
    for lib, odir, srcs, extra in variants:
        os.makedirs(odir, exist_ok=True)
        objs = [os.path.join(odir, s.replace(".hip", ".o")) for s in srcs]
        cmds += [[cc, *FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
        links.append((lib, objs))
    with ThreadPoolExecutor(max_workers=jobs or min(8, len(cmds))) as ex:
        for msg in ex.map(_run, cmds):
            if verbose and msg.strip():
                print(msg)
    for lib, objs in links:
        tmp = lib + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
