"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

The flags keep the arithmetic plain IEEE fp32: no FMA contraction, no
fast-math, SSE floating point (x86-64 default), correctly rounded division
and square root.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-std=c99", "-O2", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> str:
    """Compile oracle.c; always recompiles. Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
