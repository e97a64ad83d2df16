"""Build script for the fp64 CPU oracle (test infrastructure, not product code).

Compiles oracle.c (the fp64 oracle) and emulate.c (the precision-emulating
model of the flash and baseline algorithms) with gcc into liboracle.so next to
this file.  No fused multiply-add contraction and no fast-math, so the
arithmetic is exactly the sequence of IEEE double operations the C source
spells out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, "oracle.c"), os.path.join(HERE, "emulate.c")]
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           *srcs, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
