"""Build librfp2.so (the ROCmFP2 HIP library) for gfx950, in-tree.

Every `.hip` file under csrc/ is compiled to its own object in parallel and
the objects are linked into bit_gemv_amd/librfp2.so.  The build always
recompiles (it is the "does it build" check as well as the build).
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "rfp2")
LIB = os.path.join(HERE, "librfp2.so")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librfp2.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(jobs: int | None = None) -> str:
    """Compile every source and link librfp2.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(lambda so: _run([hipcc, *CFLAGS, "-c", so[0], "-o", so[1]]),
                      zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
