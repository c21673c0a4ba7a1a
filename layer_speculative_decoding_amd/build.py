"""Build libspec.so (all HIP sources under csrc/) for gfx950 with hipcc.

Usage: python -m layer_speculative_decoding_amd.build  (or build() from Python)
Each source is compiled to its own object (in parallel) under _build/, then
linked; the library is written next to this file so that it travels with the
tree.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspec.so")
OBJ = os.path.join(HERE, "..", "_build")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libspec.so")


def build(verbose: bool = False, extra_flags=(), lib: str = LIB) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    tag = os.path.basename(lib).replace(".so", "")
    objs = [os.path.join(OBJ, f"{tag}_{os.path.basename(s)[:-4]}.o") for s in srcs]
    cmds = [[hipcc(), *FLAGS, *extra_flags, *inc, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = min(len(cmds), max(1, min(os.cpu_count() or 1, 16)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib + ".tmp"
    _run([hipcc(), *FLAGS, *extra_flags, "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
