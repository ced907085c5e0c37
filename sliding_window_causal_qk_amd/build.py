"""Build libswattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sliding_window_causal_qk_amd.build

Every call recompiles.  The library lands next to this file; the Python
binding loads it from there.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libswattn.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags(extra=()):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed fp32 instructions on its own
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
        *extra,
    ]


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
