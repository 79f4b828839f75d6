"""Build librrb.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

``python -m reduce_rank_buffers_amd.build`` or ``build()`` compiles every
source under ``csrc/`` with hipcc for gfx950 into
``reduce_rank_buffers_amd/librrb.so``, and the same library with the chain
kernels built with RRB_SNAC_FENCES=1 (memory-model release/acquire ordering
of the SNAC flags) into ``librrb_fenced.so``.  Always recompiles.  The
sources are compiled to objects in parallel (one hipcc process each) and then
linked; device code does not call across files, so no relocatable device
code is needed.
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
LIB_FENCED = os.path.join(PKG, "librrb_fenced.so")
FENCED_SOURCE = "rrb_snac.hip"
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
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="rrb_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in srcs]
        fenced_obj = os.path.join(tmp, FENCED_SOURCE + ".fenced.o")
        jobs = [([HIPCC, *FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o], s) for s, o in zip(srcs, objs)]
        jobs.append(([HIPCC, *FLAGS, "-DRRB_SNAC_FENCES=1", *inc, "-c", os.path.join(CSRC, FENCED_SOURCE),
                      "-o", fenced_obj], FENCED_SOURCE + " (fenced)"))
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(lambda job: _run(job[0], verbose, job[1]), jobs))
        fenced_objs = [fenced_obj if s == FENCED_SOURCE else o for s, o in zip(srcs, objs)]
        for lib, lib_objs in ((LIB, objs), (LIB_FENCED, fenced_objs)):
            _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *lib_objs, "-o", lib + ".tmp"], verbose,
                 "link " + os.path.basename(lib))
    os.replace(LIB + ".tmp", LIB)
    os.replace(LIB_FENCED + ".tmp", LIB_FENCED)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
