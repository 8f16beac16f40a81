"""Builds libnq.so (the HIP library for gfx950) in-tree with hipcc.

Run ``python kv_cache_compression_proxy_amd/build.py`` (or ``__graft_entry__.build()``). It is
a plain script, run by path: importing the package loads the library, which must not be needed
to build it (a fresh checkout has none, an old build may lack newer entry points).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnq.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # fp32 arithmetic must round exactly as written (the encode decisions are compared
    # bit for bit): no contraction of a*b+c into fma unless written as fma
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    src = os.path.join(CSRC, "nq_api.hip")
    tmp = LIB + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
