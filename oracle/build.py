"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: the product library never links or loads this.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -O2 without -march=native: the library may run on a host CPU other than the
# one it was built on.  -ffp-contract=off keeps every fp operation a single
# IEEE-rounded operation, no fused multiply-adds, no fast-math.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
