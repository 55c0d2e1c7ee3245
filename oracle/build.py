"""Builds the CPU oracle (oracle.c -> liboracle.so) with gcc.

Test infrastructure: the oracle is only loaded by the test suite, the smoke
check and the bench's CPU-baseline leg.  -ffp-contract=off keeps every
multiply and add separately rounded, as the oracle's definition needs.  No
-march=native: the library may run on another host CPU.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
