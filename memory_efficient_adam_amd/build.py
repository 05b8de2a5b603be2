"""Builds libadam_mi355x.so in-tree with hipcc for gfx950.

Floating-point contraction is off (every fma in the kernels is written
explicitly, so results are reproducible operation by operation), fp32
division and square root stay correctly rounded (hipcc's default), and the
packed-fp32 instructions are disabled.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libadam_mi355x.so")
SOURCES = [os.path.join(CSRC, "adam_kernels.hip"), os.path.join(CSRC, "adam_runtime.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
