"""Build the CPU oracle library (test infrastructure only).

    python -m oracle.build        # or: python oracle/build.py

Compiles oracle.c, oracle_mx.c and oracle_i8.c with gcc into oracle/liboracle.so: -O2, no floating-point
contraction, no fast-math, OpenMP over output rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "oracle.c"), os.path.join(HERE, "oracle_mx.c"), os.path.join(HERE, "oracle_i8.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp] + SRCS + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
