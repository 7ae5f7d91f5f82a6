"""Build libfalqon.so (the HIP library for gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with:
  -ffp-contract=off   no silent fusion of a*b+c: the casts, the SGD step and
                      the proxy update's requantization are specified with
                      separate roundings, and fused multiply-adds appear only
                      where the code calls fmaf;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keep the compiler from forming packed fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfalqon.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc"] + HIP_FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = ["hipcc", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(srcs)} sources")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
