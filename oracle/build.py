"""Build the CPU oracle (test infrastructure) into oracle/liboracle_fp4.so.

Plain gcc, binary32/binary64 IEEE arithmetic with contraction disabled so
every rounding step in fp4_oracle.c happens exactly where it is written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4_oracle.c")
LIB = os.path.join(HERE, "liboracle_fp4.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
