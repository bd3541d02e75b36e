"""Build libspec.so (HIP, gfx950) in-tree with hipcc.

    python -m draft_sampling_verify_amd.build        # or build() from Python

Each source compiles to an object in parallel, then one link.  Flags:
  --offload-arch=gfx950            MI355X only
  -ffp-contract=off                no implicit FMA contraction (the tile and
                                   rescan kernels must compute identical logits)
  -target-feature -packed-fp32-ops keep the compiler from emitting packed fp32
                                   arithmetic
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspec.so")
SOURCES = ["api.hip", "propose.hip", "verify.hip", "schedule.hip", "cluster.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libspec)")


def _flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libspec.so (always rebuilds)."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        # the host pass does not know the packed-fp32 target feature; drop that note
        err = "\n".join(l for l in res.stderr.splitlines()
                        if "packed-fp32-ops" not in l or "error" in l)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
