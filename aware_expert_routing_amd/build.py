"""Build libmoe.so (HIP for gfx950) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed fp32 vector
instructions disabled.  The routing and quantiser sources additionally
disable floating-point contraction (their decisions must be bit-reproducible).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "residency.cpp", "route.hip", "ffn.hip", "quant.hip", "pack.hip", "probe.hip"]
NO_CONTRACT = {"route.hip", "quant.hip"}

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
          "-Wno-unknown-pragmas"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, src + ".o")
    cmd = [_hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj,
           "-I", os.path.join(HERE, "..", "include")]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
        cmd += ["-ffp-contract=off"] if src in NO_CONTRACT else ["-ffp-contract=fast"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so next to this file."""
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
