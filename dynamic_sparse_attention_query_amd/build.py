"""Build libdsa.so (the HIP library for gfx950) next to this file.

    python -m dynamic_sparse_attention_query_amd.build

Compiles every csrc/*.hip to an object (in parallel) and links them into one
shared library with hipcc. Always rebuilds.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdsa.so")
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 instructions stay off on this target
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core accumulators in ordinary VGPRs: the softmax and
         # max-reductions read them with vector ALU instructions, which
         # cannot address the accumulation registers directly
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile each source to an object in parallel, then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    objs = [os.path.join(objdir, os.path.basename(src)[:-4] + ".o") for src in srcs]
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, [hipcc(), *FLAGS, *inc, "-c", src, "-o", obj], verbose)
                  for src, obj in zip(srcs, objs)]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
