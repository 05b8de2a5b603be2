"""Builds the oracle's shared library (test infrastructure only).

The oracle is plain C compiled without floating-point contraction or
fast-math, so each fp32 operation it writes is rounded exactly once.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "adam_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle_adam.so")


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = [
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
        "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
        "-fPIC", "-shared", "-o", tmp, SOURCE, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
