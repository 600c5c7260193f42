"""Build the CPU oracle (test infrastructure) with gcc.

No fused multiply-add contraction and no fast-math, so every fp32 product and
sum in the oracle is a single IEEE round-to-nearest-even operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libtsv_oracle.so")
SRC = os.path.join(HERE, "tsv_oracle.c")


def build(extra_flags=()):
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", *extra_flags, "-o", LIB + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
