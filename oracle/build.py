"""Build the CPU oracle (test infrastructure) into oracle/libk3o.so with gcc.

-ffp-contract=off keeps every multiply and add separately rounded, as the
pages' engine does ("kimi-k3-in-c" README, section "The codebase").
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "k3o.c")
LIB = os.path.join(HERE, "libk3o.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=gnu11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
