"""Compile the C oracle (``zo_oracle.c``) into ``liboracle.so`` next to it.

TEST INFRASTRUCTURE ONLY: the library built here is loaded by the test suite, the smoke
check and the benchmark's CPU-baseline leg, never by the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zo_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No FMA contraction and no fast-math: the oracle's roundings are the IEEE ones the
# source spells out, one operation at a time.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
