"""Compiles the HIP sources in ``csrc/`` into ``libgs_raster.so`` for gfx950 (in-tree, so it ships with the repo)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgs_raster.so")
SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
# calibration kernels for the benchmark's counter and issue-rate checks (a separate library, not the ABI)
CALIB_LIB = os.path.join(HERE, "libgs_calib.so")
CALIB_SOURCES = [os.path.join(HERE, "csrc", "calib", "valu_calib.hip")]
HEADERS = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hpp"))) + [os.path.join(ROOT, "include", "gs_raster.h")]

# -ffp-contract=off: the composite's float32 operation order is part of its definition (no fused multiply-adds
# except the ones the source writes). Packed FP32 instructions are disabled for the whole library.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def stale() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(CALIB_LIB):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(CALIB_LIB))
    return any(os.path.getmtime(f) > t for f in SOURCES + CALIB_SOURCES + HEADERS)


def _compile(sources, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(CALIB_SOURCES, CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
