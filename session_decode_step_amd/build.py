"""Build libkd.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m session_decode_step_amd.build`` (or ``__graft_entry__.build()``).
Every source is compiled on each call; objects go to ``session_decode_step_amd/_build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkd.so")
ARCH = "gfx950"
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

# -ffp-contract=off: every fused multiply-add in the kernels is written out (fmaf), so the
# fp32 operation sequence of each output is the one in the source, whatever B is.
# -packed-fp32-ops off: no packed fp32 instructions are generated.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", f"-I{INCLUDE}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True, out: str = LIB, build_dir: str = BUILD, extra=()) -> str:
    """Compile every source (``extra``: additional hipcc flags) and link ``out``."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    LIBP = out
    tmp = LIBP + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIBP)
    if verbose:
        print(f"built {LIBP} from {len(srcs)} sources")
    return LIBP


if __name__ == "__main__":
    build()
