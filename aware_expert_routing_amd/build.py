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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (CPU checks of
# the ABI validation, pools, budget tracker and policy; the device code is
# built as usual).  Each -fsanitize= applies to the host pass only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
ASAN_DIR = os.path.join(OUT_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libmoe.so")


def _compile(src: str, out_dir: str = OUT_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, src + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj,
           "-I", os.path.join(HERE, "..", "include")]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
        cmd += ["-ffp-contract=off"] if src in NO_CONTRACT else ["-ffp-contract=fast"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link libmoe.so next to this file; with
    sanitize=True, a host-sanitized copy in _build/asan/ instead (load it with
    MOE_LIB=<path> and the sanitizer runtime preloaded)."""
    out_dir, lib, extra = (ASAN_DIR, ASAN_LIB, SANITIZE_HOST) if sanitize else (OUT_DIR, LIB, [])
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
