"""Build the HIP library ``libkdn.so`` (gfx950) in-tree with hipcc.

Usage: ``python -m kalman_delta_rule_amd.build`` (also called by the repo's
``__graft_entry__.build()``).  The library is placed next to this file so it
travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkdn.so")
SOURCES = ["kdn_api.cpp", "kdn_walk.hip", "kdn_chunk.hip", "kdn_step.hip", "kdn_gain.hip",
           "kdn_dense.hip", "kdn_bwd.hip", "kdn_bwd_chunk.hip",
           "kdn_prologue.hip", "kdn_seqpar.hip", "kdn_plan.cpp"]
# sources whose kernels use the matrix cores (checked by isa_check)
MFMA_SOURCES = ["kdn_walk.hip", "kdn_chunk.hip", "kdn_bwd_chunk.hip"]
ARCH = os.environ.get("KDN_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build_library(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ([hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
           + srcs + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkdn.so")
    probs = run_isa_check(verbose=verbose)
    if probs:
        sys.stderr.write("\n".join(probs) + "\n")
        os.unlink(tmp)
        raise RuntimeError("matrix-core dependency check failed (see isa_check.py)")
    os.replace(tmp, LIB)
    return LIB


def run_isa_check(verbose: bool = False):
    """Scan the device assembly for matrix-core dependencies the compiler
    does not pad (isa_check.py); returns the list of problems."""
    from kalman_delta_rule_amd import isa_check
    return isa_check.check_sources([os.path.join(CSRC, s) for s in MFMA_SOURCES],
                                   [os.path.join(ROOT, "include"), CSRC], hipcc(),
                                   HIPCC_FLAGS, verbose=verbose)


if __name__ == "__main__":
    print(build_library(verbose=True))
