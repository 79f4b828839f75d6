"""Build librrb.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

``python -m reduce_rank_buffers_amd.build`` or ``build()`` compiles every
source under ``csrc/`` with hipcc for gfx950 into
``reduce_rank_buffers_amd/librrb.so``.  Always recompiles.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "librrb.so")
SOURCES = ["rrb_capi.cpp", "rrb_plan.cpp", "rrb_atom.hip", "rrb_moe.hip", "rrb_snac.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # bit-exact arithmetic: no contraction into FMA, IEEE denormals kept
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose=False):
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("librrb build failed")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
