"""Builds the CPU oracle (test infrastructure) into oracle/libdro.so with gcc.

The flags keep every operation a single IEEE fp32 operation: no contraction of
a*b+c into an fma (every fma in the oracle is an explicit fmaf call), no
fast-math, no flush of subnormals.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libdro.so")


FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
         "-fPIC", "-shared", "-Wall", "-Wextra", "-pthread"]


def compile_source(src: str, out: str) -> str:
    """Compile one oracle source file (with dro.h beside it) into `out`."""
    subprocess.run(["gcc"] + FLAGS + [src, "-o", out, "-lm"], check=True)
    return out


def build(verbose: bool = False) -> str:
    cmd = ["gcc"] + FLAGS + [os.path.join(HERE, "dro.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
