"""Build the HIP library libqmoe.so for gfx950 in-tree (hipcc, no torch).

    python -m quantized_moe_expert_route_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(LIB_DIR, "libqmoe.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every kernel source for gfx950 and link libqmoe.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(LIB_DIR, exist_ok=True)
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
        if verbose and out.strip():
            print(out)
        return obj

    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


PROBE_SRC = os.path.join(ROOT, "tests", "probe", "mfma_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "probe", "libmfma_probe.so")


def build_probe() -> str:
    """Compile the MFMA characterization probe the GPU tests load (test
    infrastructure, not part of libqmoe.so)."""
    if not os.path.exists(PROBE_SRC):
        return ""
    cmd = [_hipcc(), *FLAGS, "-shared", PROBE_SRC, "-o", PROBE_LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe build failed:\n" + r.stdout + r.stderr)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


def resource_usage() -> dict:
    """Per-kernel register and scratch use of this build, from the compiler's
    kernel-resource-usage remarks: {kernel: {"VGPRs": .., "AGPRs": ..,
    "ScratchSize": .., "Occupancy": ..}}."""
    import re

    hipcc = _hipcc()
    usage = {}
    for src in sources():
        cmd = [hipcc, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(r.stderr)
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = m.group(1)
                usage[cur] = {}
                continue
            m = re.search(r"remark: +([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
            if cur and m:
                usage[cur][m.group(1).replace(" ", "")] = int(m.group(2))
    return usage


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe())
