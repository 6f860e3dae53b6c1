"""Builds libdsa.so (all HIP sources of the path, gfx950) and the
benchmark's measurement probe libdsa_bench.so in-tree with hipcc.

Every call recompiles.  Objects go to _build/ next to this file; the shared
libraries land beside this file, where the binding (and bench.py) load them.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa.so")
BENCH_LIB = os.path.join(HERE, "libdsa_bench.so")
ARCH = "gfx950"
SOURCES = ["abi.hip", "index_scores.hip", "topk.hip", "sparse_attn.hip", "spec_verify.hip"]
BENCH_SOURCES = ["bench_peak.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 arithmetic stays off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    cmds = []

    def objs_of(sources):
        out = []
        for src in sources:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            out.append(obj)
            cmds.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return out

    lib_objs, bench_objs = objs_of(SOURCES), objs_of(BENCH_SOURCES)
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for target, objs in ((LIB, lib_objs), (BENCH_LIB, bench_objs)):
        tmp = target + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, target)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
