"""Build the CPU oracle library (test infrastructure only).

``python -m oracle.build`` or ``build()`` compiles ``bsoracle.c`` with gcc into
``oracle/libbsoracle.so``.  No fast-math and no floating-point contraction:
the oracle's fp32 steps must be exactly the IEEE operations its source names.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bsoracle.c")
LIB = os.path.join(HERE, "libbsoracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose=False):
    cmd = ["gcc"] + CFLAGS + [SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
