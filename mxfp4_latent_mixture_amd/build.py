"""Build the HIP library liblmoe.so for gfx950 (MI355X), in-tree.

Run as `python mxfp4_latent_mixture_amd/build.py` (a plain script, so it does not
import the package, whose import needs the built library). The library is written next
to this file; the Python binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "liblmoe.so")
SOURCES = ["api.hip", "route.hip", "experts.hip", "decode.hip", "decode_multi.hip", "packed.hip", "dense.hip",
           "measure.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build liblmoe.so")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 into liblmoe.so; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed-fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # single-lane atomics stay as written: the atomic optimizer would turn
        # a ticket draw into one whose result is read back at once
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-I", INCLUDE, "-o", tmp,
    ] + [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        sys.stdout.write(res.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
