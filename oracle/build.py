"""Build the oracle's one C file (oracle/chain.c) into oracle/liborchain.so.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle).
Plain gcc, -O2, no fast-math, no contraction of a*b+c into fused
multiply-adds (the only fused multiply-adds are the explicit fmaf calls).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "chain.c")
    out = os.path.join(HERE, "liborchain.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
