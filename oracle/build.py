"""Build the CPU oracle library (test infrastructure; see mx_oracle.c).

gcc, plain C11, -O2 with FP contraction off and no fast-math, OpenMP for the
outer loops only.  Writes oracle/libmxoracle.so next to this file.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mx_oracle.c")
LIB = os.path.join(HERE, "libmxoracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build_oracle(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose="-v" in sys.argv))
