"""The C ABI used from plain C99 (tests/capi_demo.c, built by
__graft_entry__.build()): no Python binding, no torch. On the CPU the program
runs its host-side part (argument errors, layout queries against the C
oracle); on the GPU it runs copy-in, three fused steps over every rank and a
gather, bit for bit against the oracle."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import __graft_entry__  # noqa: E402


def demo():
    __graft_entry__.ensure_built()
    return __graft_entry__.CAPI_DEMO


def test_host_side_from_c():
    res = subprocess.run([demo(), "--host-only"], stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, timeout=60)
    out = res.stdout.decode(errors="replace")
    assert res.returncode == 0 and "host checks ok" in out, out


@pytest.mark.gpu
def test_step_and_gather_from_c():
    print("[capi_demo] full run", flush=True)
    res = subprocess.run([demo()], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         timeout=100)
    out = res.stdout.decode(errors="replace")
    assert res.returncode == 0 and "capi demo ok" in out, out
