"""Build step of libfsdppack: compile the HIP kernels and the host code for
gfx950 with hipcc into ``libfsdppack.so`` next to this file (in-tree, so the
built library travels with the source tree)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfsdppack.so")
ARCH = "gfx950"

SOURCES = ["fsdppack_kernels.hip", "fsdppack_plan.cpp", "fsdppack_abi.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libfsdppack")


def command(out: str = LIB) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wextra", "-Wno-unused-parameter",
            # no packed-fp32 instructions in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the pack kernel's six leading scalar arguments (its direct test's
            # inputs) are placed in scalar registers before each wave starts
            # (with a fallback that loads them on firmware without preloading)
            "-mllvm", "-amdgpu-kernarg-preload-count=6",
            "-I", os.path.join(HERE, "..", "include"),
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False) -> str:
    """Compile libfsdppack.so (always recompiles).  Returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-6000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
