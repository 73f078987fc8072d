"""Build the oracle's C arithmetic into oracle/liboracle.so (test infrastructure).

gcc, -O2 -ffp-contract=off and no fast-math: every float operation in step.c is
one IEEE-754 binary32 operation rounded to nearest-even, subnormals kept.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "step.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
          "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False, src: str = SRC, out: str = LIB, werror: bool = True) -> str:
    tmp = out + ".tmp"
    flags = CFLAGS if werror else [f for f in CFLAGS if f != "-Werror"]
    cmd = ["gcc", *flags, src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
