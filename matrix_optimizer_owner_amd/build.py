"""Build the gfx950 HIP library libmfsdp.so in-tree with hipcc.

Usage: python -m matrix_optimizer_owner_amd.build   (or build() from Python)
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmfsdp.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["plan.cpp", "owner_planner.cpp", "checkpoint.cpp", "step.hip", "elementwise.hip", "ns_gemm.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmfsdp.so)")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libmfsdp.so next to this file.
    Always recompiles.  Returns the library path."""
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    common = [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # no packed-fp32 instructions anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(obj_dir, src + ".o")
        lang = ["-x", "c++"] if src.endswith(".cpp") else ["-x", "hip"]
        cmd = [cc, *common, *lang, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libmfsdp.so failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
