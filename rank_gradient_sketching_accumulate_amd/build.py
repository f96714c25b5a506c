"""Build liblogra.so (HIP, gfx950) in-tree with hipcc.

Run ``python -m rank_gradient_sketching_accumulate_amd.build`` or call
``build_library()``.  The library is always rebuilt when this is called:
every translation unit is compiled to an object in parallel, then the
objects are linked into one shared library.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
LIB_NAME = "liblogra.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"
# hipcc's host pass warns that it does not know the packed-fp32 feature.
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-munsafe-fp-atomics",
        # Keep the compiler from forming packed fp32 arithmetic.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(REPO_DIR, "include"),
        "-Wall",
        "-Wno-unused-function",
    ]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    return res.returncode, err


def build_library(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="logra_build_") as od:
        objs = [os.path.join(od, os.path.basename(s)[:-4] + ".o") for s in SOURCES]
        cmds = [[hipcc(), *compile_flags(), "-c", s, "-o", o] for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "8"))))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for c, (rc, err) in zip(cmds, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {c[-3]}:\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
