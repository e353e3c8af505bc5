"""Build libhaste.so (HIP, gfx950) in-tree with hipcc.

Each .hip source under csrc/ is compiled to an object file in parallel, then
linked into group_shared_fixed_amd/libhaste.so.  hipcc cross-compiles for
gfx950 without a GPU present.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libhaste.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libhaste.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-L/opt/rocm/lib", "-lrocblas",
           "-Wl,-rpath,/opt/rocm/lib", f"-Wl,--version-script={os.path.join(CSRC, 'exports.map')}"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
