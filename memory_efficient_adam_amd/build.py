"""Builds libadam_mi355x.so (the step) and libadam_stream_probe.so (the
stream probe, a measurement kernel the step does not use) in-tree with hipcc
for gfx950.

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
PROBE_LIBRARY = os.path.join(HERE, "libadam_stream_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "stream_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _build_one(library, sources, verbose):
    tmp = library + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, library)


def build(verbose: bool = False) -> str:
    _build_one(LIBRARY, SOURCES, verbose)
    _build_one(PROBE_LIBRARY, PROBE_SOURCES, verbose)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
