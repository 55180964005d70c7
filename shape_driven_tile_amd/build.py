"""Build libsdt.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m shape_driven_tile_amd.build [--resource-usage]
    python -m shape_driven_tile_amd.build --resource-summary PATH

Writes ``shape_driven_tile_amd/libsdt.so``.  With ``--resource-usage`` the
compiler's per-kernel register/LDS/spill report is printed as well;
``--resource-summary PATH`` writes that report as a markdown table instead of
building the library.
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
    write_build_info()
    return LIB


BUILD_INFO = os.path.join(HERE, "build_info.json")


def write_build_info() -> None:
    """Record what libsdt.so was built from (the git commit and whether the
    tree had uncommitted changes, the compiler's version line) beside it, for
    the benchmark's receipt; fields that cannot be read are null."""
    import json

    def run(cmd):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=30)
            return r.stdout.strip() if r.returncode == 0 else None
        except (OSError, subprocess.SubprocessError):
            return None
    status = run(["git", "status", "--porcelain", "--untracked-files=no"])
    hip = run([hipcc(), "--version"])
    info = {"commit": run(["git", "rev-parse", "HEAD"]),
            "dirty": None if status is None else bool(status),
            "hipcc": hip.splitlines()[0] if hip else None,
            "arch": ARCH}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


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


def resource_summary(path: str) -> str:
    """Compile the library with the compiler's per-kernel resource remarks and
    write them as a markdown table (one row per kernel instantiation:
    registers, spills, LDS, occupancy) to `path`."""
    import re
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS + [
           "-Rpass-analysis=kernel-resource-usage", "--cuda-device-only", "-c",
           os.path.join(CSRC, "sdt.hip"), "-o", os.devnull]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    rows, cur = [], None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"mangled": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]*\])?: (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    names = subprocess.run(["c++filt"], input="\n".join(r["mangled"] for r in rows),
                           capture_output=True, text=True).stdout.splitlines()
    out = ["# Kernel resources: every instantiation in libsdt.so (gfx950)", "",
           "The compiler's own report (`-Rpass-analysis=kernel-resource-usage`) for the",
           "device code of `shape_driven_tile_amd/csrc/sdt.hip`, written by", "",
           "    python -m shape_driven_tile_amd.build --resource-summary "
           "profiles/kernel_resource_usage.md", "",
           "VGPRs and AGPRs are per lane (the two files are allocated together on",
           "gfx950: 512 per SIMD lane in all, so a wave using V + A registers leaves",
           "room for floor(512 / (V + A)) waves per SIMD, at most 8); LDS is per workgroup",
           "(160 KB per CU).", "",
           "| kernel | VGPRs | AGPRs | SGPRs | VGPR spill | SGPR spill | scratch B/lane | LDS bytes | waves/SIMD |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r, n in zip(rows, names):
        n = n.replace("void ", "").replace("sdt::(anonymous namespace)::", "sdt::")
        n = re.sub(r"\(.*\)$", "", n)
        out.append(f"| `{n}` | {r.get('VGPRs', '?')} | {r.get('AGPRs', '?')} | "
                   f"{r.get('TotalSGPRs', '?')} | {r.get('VGPRs Spill', '?')} | "
                   f"{r.get('SGPRs Spill', '?')} | {r.get('ScratchSize', '?')} | "
                   f"{r.get('LDS Size', '?')} | {r.get('Occupancy', '?')} |")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    return path


if __name__ == "__main__":
    if "--resource-summary" in sys.argv:
        print(resource_summary(sys.argv[sys.argv.index("--resource-summary") + 1]))
        sys.exit(0)
    build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv)
    print(LIB)
