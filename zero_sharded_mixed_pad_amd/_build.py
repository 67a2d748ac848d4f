"""Compile libzsp.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

The library is built next to this file so that it travels with the source
tree; nothing is installed. Device-code flags:
  -ffp-contract=off     the Adam arithmetic must not be fused into FMAs
  -packed-fp32-ops off  no v_pk_*_f32 instructions are generated
Division and square root keep HIP's default correctly rounded expansions.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzsp.so")

ARCH = "gfx950"
SOURCES = ["zsp_kernels.hip", "zsp_capi.cpp", "zsp_layout.cpp", "zsp_gather_list.cpp",
           "zsp_noalloc.hip", "zsp_ckpt.cpp", "zsp_ckpt_dev.cpp", "zsp_sched.cpp"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; libzsp needs ROCm's hipcc to build")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every source into libzsp.so; always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    out = res.stdout.decode(errors="replace")
    # hipcc's host pass does not know the device-only feature; that note is noise.
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
