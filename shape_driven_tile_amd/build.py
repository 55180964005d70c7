"""Build libsdt.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m shape_driven_tile_amd.build [--resource-usage]

Writes ``shape_driven_tile_amd/libsdt.so``.  With ``--resource-usage`` the
compiler's per-kernel register/LDS/spill report is printed as well.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsdt.so")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "sdt.hip"), os.path.join(CSRC, "launcher.cpp")]

# Packed fp32 vector ops are switched off for every device compile.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if (resource_usage or verbose) and err:
        print(err)
    os.replace(tmp, LIB)
    return LIB


CAPI_SRC = os.path.join(ROOT, "tests", "capi", "capi_check.cpp")
CAPI_BIN = os.path.join(ROOT, "tests", "capi", "capi_check")


def build_capi_check() -> str:
    """The C-ABI test program (host code only): links libsdt.so and the CPU
    oracle's libsdt_oracle.so, found next to it through an $ORIGIN rpath."""
    tmp = CAPI_BIN + ".tmp"
    cmd = [hipcc(), "-O2", "-std=c++17", "-Wall", "-I", INCLUDE, CAPI_SRC, "-o", tmp,
           "-L", HERE, "-lsdt", "-L", os.path.join(ROOT, "oracle"), "-lsdt_oracle",
           "-Wl,-rpath,$ORIGIN/../../shape_driven_tile_amd:$ORIGIN/../../oracle"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, CAPI_BIN)
    return CAPI_BIN


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv)
    print(LIB)
