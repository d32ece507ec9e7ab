"""Builds libspec.so (the HIP library behind include/spec.h) in-tree for gfx950.

    python -m speculative_decoding_token_amd.build [--debug]

Each source is compiled to an object of its own (in parallel), then the objects are linked.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspec.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {cmd[-1]}")


def build(verbose: bool = False, debug: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-O1" if debug else "-O3",
             # no packed-fp32 instructions anywhere in the library
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc] + flags + ["-c", "-o", obj, src])
    workers = min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    out_tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + objs, verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv))
