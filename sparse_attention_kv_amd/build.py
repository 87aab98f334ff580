"""Build libflashloop.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU
instructions disabled; the quantiser and selection sources are additionally
compiled without multiply-add contraction (their codes and scales must be
reproducible bit for bit)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflashloop.so")

SOURCES = ["abi.hip", "select.hip", "quant.hip", "attn.hip", "adaptive.hip", "block.hip", "decode.hip",
           "calib.hip"]
NO_CONTRACT = {"select.hip", "quant.hip"}
# the precision-adaptive attention's fused rebuild + attention instantiation
# exceeds the default inlining budget (its per-tile lambdas would become
# device-function calls with a stack frame); the other instantiations
# compile to the same code with or without this
EXTRA = {"adaptive.hip": ["-mllvm", "-inline-threshold=5000"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    flags = list(COMMON)
    if src in NO_CONTRACT:
        flags.append("-ffp-contract=off")
    flags += EXTRA.get(src, [])
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
