"""Build librrb.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

``python -m reduce_rank_buffers_amd.build`` or ``build()`` compiles every
source under ``csrc/`` with hipcc for gfx950 into
``reduce_rank_buffers_amd/librrb.so``.  Always recompiles.  The sources are
compiled to objects in parallel (one hipcc process each) and then linked;
device code does not call across files, so no relocatable device code is
needed.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "librrb.so")
SOURCES = ["rrb_capi.cpp", "rrb_plan.cpp", "rrb_atom.hip", "rrb_moe.hip", "rrb_snac.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # bit-exact arithmetic: no contraction into FMA, IEEE denormals kept
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("librrb build failed: " + what)
    # warnings are shown, not hidden
    if res.stderr.strip():
        sys.stderr.write(res.stderr)
    return res


def build(verbose=False):
    srcs = SOURCES
    with tempfile.TemporaryDirectory(prefix="rrb_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in srcs]
        cmds = [[HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
                 os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
        workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(lambda cs: _run(cs[0], verbose, cs[1]), zip(cmds, srcs)))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose,
             "link")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
