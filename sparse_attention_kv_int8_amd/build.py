"""Builds libsd.so (the HIP library behind include/sd.h) for gfx950, in-tree.

    python -m sparse_attention_kv_int8_amd.build [--verbose]
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsd.so")
ARCH = os.environ.get("SD_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # correctly rounded fp32 division: the int8 codes depend on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return h


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compiles every source into libsd.so (atomically replaced)."""
    srcs = sources()
    fd, tmp = tempfile.mkstemp(prefix="libsd.", suffix=".so.tmp", dir=PKG)
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-8000:]}")
    if verbose and r.stderr.strip():
        print(r.stderr[-4000:], file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
