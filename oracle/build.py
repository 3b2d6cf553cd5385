"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with gcc.

The flags keep every float operation IEEE binary32 round-to-nearest-even:
no FMA contraction, no fast-math.  OpenMP only threads the fp64 GEMM
reference over independent outputs.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp,
           "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
