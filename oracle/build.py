"""Compile the oracle (plain C, host only) into oracle/liboracle.so with gcc.

Test infrastructure: the result is loaded only by the tests, the package smoke
check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, every product and sum rounds once
# as written.  -fno-fast-math keeps IEEE semantics (division, NaN, signed 0).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
          "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
          "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
