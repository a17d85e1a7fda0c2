"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

The oracle is compiled without fast-math and without FMA contraction, so every
operation written in oracle.c is one IEEE double operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = [os.path.join(HERE, "oracle.c"), os.path.join(HERE, "decoder.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    srcs = [s for s in SRC if os.path.exists(s)]
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas",
           *srcs, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
