"""The checkpoint file module (zsp_ckpt.cpp) under AddressSanitizer and
UBSan (CPU only): rank files written, checked and mapped, then truncated,
bit-flipped and hostile files, each of which must be refused without any
out-of-bounds access or oversized allocation ("ZeRO Stages: Sharding
Optimizer State, Gradients, and Parameters", "Where the shards live and what
happens on failure"). The driver is tests/ckpt_check.cpp."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_mixed_pad_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_checkpoint_files_under_sanitizers(tmp_path):
    exe = str(tmp_path / "ckpt_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(ROOT, "tests", "ckpt_check.cpp"),
                    os.path.join(CSRC, "zsp_ckpt.cpp"), "-o", exe], check=True)
    work = tmp_path / "ckpt"
    work.mkdir()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe, str(work)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         timeout=300, env=env)
    out = res.stdout.decode(errors="replace")
    assert res.returncode == 0 and out.strip().endswith("ok"), out[-3000:]
