"""Build libspecverify.so in-tree with hipcc for gfx950.

Usage: ``python -m speculative_decoding_sampling_amd.build`` (or
``__graft_entry__.build()``).  Compiles every source under ``csrc/`` to an
object in ``_build/`` in parallel and links the shared library next to this
file, where the Python binding loads it.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libspecverify.so")

ARCH = "gfx950"
SOURCES = ["specverify.hip", "row_stats.hip", "accept.hip", "sample.hip", "filter.hip",
           "filter_rows.hip", "sample_list.hip", "diagnostics.hip", "round_policy.hip",
           "lm_head.hip", "small.hip"]
# Packed FP32 instructions stay off: the compiler must not form v_pk_* FP32 ops.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libspecverify)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose=False):
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
