"""Compile the oracle's C into oracle/liboracle.so with gcc.

The oracle is test infrastructure, not part of the product path.

    python oracle/build_oracle.py
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# x86-64 SSE scalar arithmetic, no FMA contraction, no fast-math
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
