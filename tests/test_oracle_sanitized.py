"""The oracle's pin suite run against the oracle built under
AddressSanitizer and UBSan (CPU only): every pin must still pass, and any
out-of-bounds access, use after free, overflow or other undefined behaviour
in oracle.c ends the run with a report instead."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
PINS = ["tests/test_oracle_layout.py", "tests/test_oracle_reduce.py",
        "tests/test_oracle_adam.py", "tests/test_oracle_stages.py",
        "tests/test_oracle_brute.py"]


def asan_runtime():
    if shutil.which("gcc") is None:
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(asan_runtime() is None, reason="needs gcc with libasan")
def test_oracle_pins_under_sanitizers(tmp_path):
    from oracle import build as oracle_build
    lib = oracle_build.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    nm = subprocess.run(["nm", "-D", lib], stdout=subprocess.PIPE, text=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm, "the build is not instrumented"
    env = dict(os.environ, ZSP_ORACLE_LIB=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", *PINS], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, timeout=900)
    out = res.stdout.decode(errors="replace")
    assert res.returncode == 0, out[-3000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
