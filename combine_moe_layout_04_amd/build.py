"""Build libmoe_layout.so for gfx950 with hipcc, in-tree.

Flags: -O3, no fused multiply-add contraction (the float32 contract rounds
every product and sum on its own), packed-fp32 instructions disabled, C++17.
Each source is compiled to an object in parallel, then linked.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_layout.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["abi.hip", "layout_kernels.hip", "row_kernels.hip", "staged_kernels.hip", "copy_kernels.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-I", INCLUDE,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


C_ABI_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "moe_c_abi_check.cpp")
C_ABI_CHECK = os.path.join(ROOT, "tests", "c_abi", "moe_c_abi_check")


def build_c_abi_check() -> str:
    """The C++ program that drives the library through its C ABI alone (no
    Python, no torch), linked against the in-tree library; returns its path."""
    _run([hipcc(), f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-I", INCLUDE, C_ABI_CHECK_SRC,
          "-o", C_ABI_CHECK, "-L", PKG, "-lmoe_layout", "-Wl,-rpath,$ORIGIN/../../combine_moe_layout_04_amd"])
    return C_ABI_CHECK


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library (then the C ABI
    check program against it); returns the library's path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    build_c_abi_check()
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
