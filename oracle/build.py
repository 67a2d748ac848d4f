"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

The flags keep the arithmetic plain IEEE fp32: no FMA contraction, no
fast-math, SSE floating point (x86-64 default), correctly rounded division
and square root. build(sanitize=True) (or `python oracle/build.py
--sanitize`) builds the same source under AddressSanitizer and UBSan
instead, into oracle/liboracle_san.so; a process that loads it needs the
ASan runtime preloaded (LD_PRELOAD of gcc's libasan.so).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
LIB_SAN = os.path.join(HERE, "liboracle_san.so")

CFLAGS = [
    "-std=c99", "-O2", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra",
]


SANFLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    """Compile oracle.c; always recompiles. Returns the library path."""
    lib = out or (LIB_SAN if sanitize else LIB)
    tmp = lib + ".tmp"
    flags = CFLAGS + (SANFLAGS if sanitize else [])
    cmd = ["gcc", *flags, "-o", tmp, os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
