"""Build libmoe.so in-tree for gfx950 with hipcc (no JIT, no caches outside the repo)."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
# the same sources with -DMOE_DEBUG: kernels record invariant violations in
# the workspace and moe_drop_stats reports them (MOE_ECAP); nothing traps
LIB_DEBUG = os.path.join(PKG, "libmoe_debug.so")
SOURCES = ["kernels.hip", "api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off: hipcc would otherwise form v_pk_* from float2 code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, extra_flags=()):
    """Build libmoe.so and its debug twin libmoe_debug.so (-DMOE_DEBUG)."""
    variants = [(LIB, BUILD, ()), (LIB_DEBUG, os.path.join(BUILD, "debug"), ("-DMOE_DEBUG",))]
    jobs = []
    for _, bdir, flags in variants:
        os.makedirs(bdir, exist_ok=True)
        for src in SOURCES:
            jobs.append((src, os.path.join(bdir, os.path.splitext(src)[0] + ".o"), flags))

    def compile_one(job):
        src, obj, flags = job
        return _run([HIPCC, *FLAGS, *flags, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])

    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        logs = list(ex.map(compile_one, jobs))
    for lib, bdir, _ in variants:
        objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        tmp = lib + ".tmp"
        logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-o", tmp, *objs]))
        os.replace(tmp, lib)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
