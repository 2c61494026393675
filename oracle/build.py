"""Build the CPU oracle shared library (test infrastructure only).

``python -m oracle.build`` or ``oracle.build.build()`` compiles
``nabla_oracle.c`` with gcc into ``liborc_nabla.so`` next to this file.
Floating-point contraction is off: the only fused multiply-adds are the
explicit ``fmaf`` calls in the source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nabla_oracle.c")
LIB = os.path.join(HERE, "liborc_nabla.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
