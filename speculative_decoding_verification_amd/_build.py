"""Build libspecverify.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with fp contraction off (the
fused multiply-adds the kernels want are written out explicitly) and packed
fp32 instructions disabled.  matvec_inst.hip holds the projection and pass
kernels for one number of positions and is compiled once per M (1..16), so
the variants build in parallel.  Objects go to _build/; the shared library
lands next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libspecverify.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


INST = os.path.join(CSRC, "matvec_inst.hip")
MAX_M = 16


def sources():
    """(source, object name, extra defines) of every compile job."""
    jobs = [(s, os.path.basename(s) + ".o", []) for s in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
            if s != INST]
    # The kernel keeps a ring of weight records in named registers filled by
    # one load path for every format.  LLVM's sinking of common instructions
    # out of the per-format address branches would merge stores to different
    # ring registers into one store through a selected pointer, which forces
    # the ring into scratch memory; it is switched off for this file.  The
    # largest M first: they take longest.
    inst_flags = ["-mllvm", "-simplifycfg-sink-common=false"]
    jobs = [(INST, f"matvec_inst_m{m}.o", [f"-DSV_INST_M={m}", *inst_flags]) for m in range(MAX_M, 0, -1)] + jobs
    return jobs


def _compile(job, extra) -> str:
    src, name, defs = job
    obj = os.path.join(BUILD, name)
    cmd = [HIPCC, *FLAGS, *defs, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=(), link_extra=()) -> str:
    """extra: more compile flags; link_extra: more link flags (a host-side
    sanitizer build passes its runtime here)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
