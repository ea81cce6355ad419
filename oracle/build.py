"""Build the CPU oracle (liboracle.so) with gcc.

Test infrastructure only: the oracle is loaded by the test suite, the smoke
check and the bench's CPU-baseline leg, never by the GPU product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
