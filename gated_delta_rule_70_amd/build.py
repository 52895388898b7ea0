"""Build ``libgdr.so`` (the HIP library behind include/gdr.h) for gfx950 with hipcc.

Run ``python -m gated_delta_rule_70_amd.build`` (or ``__graft_entry__.build()``). It always
recompiles. Objects go to ``_build/`` at the repository root; the library is written next
to this file so that it travels with the package.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdr.so")

SOURCES = ["gdr_api.cpp", "chunk_fwd.hip", "chunk_fwd_fast.hip", "decode.hip", "gdn2_fwd.hip", "gdn2_decode.hip", "bwd.hip",
           "scratch.hip"]
ARCH = os.environ.get("GDR_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=%s" % ARCH,
            # packed fp32 instructions are switched off for all device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-core accumulators in ordinary VGPRs: the kernels apply VALU ops to
            # them every chunk, and AGPR accumulators would need a move each way
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=%s" % ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built %s" % LIB)
    return LIB


if __name__ == "__main__":
    build()
