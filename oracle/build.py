"""Build the CPU oracle's shared library (test infrastructure only).

The oracle is plain C compiled by gcc with IEEE semantics: no fast-math and
no FMA contraction, so every float operation rounds once, to nearest-even.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bsr_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
    "-fno-finite-math-only", "-frounding-math", "-fopenmp", "-fPIC", "-shared",
]


def build(verbose: bool = False) -> str:
    """Compile oracle/bsr_oracle.c into oracle/liboracle.so and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
