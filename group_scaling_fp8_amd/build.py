"""Builds libmgs.so, the gfx950 HIP library, in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmgs.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU forms anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


LIB_TRACE = os.path.join(PKG, "libmgs_trace.so")


def build(verbose: bool = False, trace: bool = False) -> str:
    """Compiles every HIP source into group_scaling_fp8_amd/libmgs.so; with
    trace=True into libmgs_trace.so instead, the same library with the dim0
    tile timeline recorded (MGS_TILE_TRACE, a diagnostic)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = LIB_TRACE if trace else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + (["-DMGS_TILE_TRACE"] if trace else []) + \
        ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, err))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
