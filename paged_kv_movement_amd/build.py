"""Build libkvmove.so for gfx950 with hipcc, in-tree (next to this file).

    python -m paged_kv_movement_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "kvmove.hip")
LIB = os.path.join(HERE, "libkvmove.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
# No fast-math: the fp8 path relies on IEEE float32 division and products.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_c_example(out: str | None = None) -> str:
    """Compile tests/abi_c_example.c, a plain C program using the C ABI,
    against libkvmove.so (found through the rpath, relative to the program
    first, then by this tree's absolute path).  The HIP
    headers need the platform macro that hipcc defines only for HIP sources."""
    src = os.path.join(ROOT, "tests", "abi_c_example.c")
    out = out or os.path.join(ROOT, "tests", "abi_c_example")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-o", tmp, src, "-L", HERE, "-lkvmove", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../paged_kv_movement_amd", "-Wl,-rpath," + HERE]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
