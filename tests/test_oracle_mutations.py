"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case rewrites one line of a copy of oracle/oracle.c into a plausible
mistake (a dropped or swapped term, a wrong sign, index or order, a missing
mask), builds the copy with the oracle's own flags, and runs the pin tests
against it in a child process. The pins pass on the real oracle, so every
case here must make them fail; a case that passes would mean the pins
cannot tell that mistake from the real definition.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")
sys.path.insert(0, ROOT)
from oracle.build import CFLAGS  # noqa: E402

LAYOUT = "tests/test_oracle_layout.py"
REDUCE = "tests/test_oracle_reduce.py"
ADAM = "tests/test_oracle_adam.py"
STAGES = "tests/test_oracle_stages.py"
BRUTE = "tests/test_oracle_brute.py"

MUTANTS = [
    ("stage 1 shards the gradients too", "const int64_t grads_n = stage >= 2 ? shard_elems : psi;",
     "const int64_t grads_n = stage >= 1 ? shard_elems : psi;", STAGES),
    ("stage 3 keeps the parameter replica", "const int64_t params_n = stage >= 3 ? shard_elems : psi;",
     "const int64_t params_n = psi;", STAGES),
    ("stage 2 all-reduces", "case 2: return reduce_scatter + all_gather;",
     "case 2: return all_reduce + all_gather;", STAGES),
    ("stage 3 gathers once", "case 3: return reduce_scatter + 2.0 * all_gather;",
     "case 3: return reduce_scatter + all_gather;", STAGES),
    ("pad even when divisible",
     "return rem == 0 ? 0 : (int64_t)nd - rem;", "return (int64_t)nd - rem;", LAYOUT),
    ("full layout forgets the pad",
     "full_off[t + 1] = full_off[t] + padded;", "full_off[t + 1] = full_off[t] + numel[t];",
     LAYOUT),
    ("interleaved instead of contiguous slices",
     "int64_t k = (int64_t)r * s + i;\n                int64_t e = base",
     "int64_t k = i * nd + r;\n                int64_t e = base", LAYOUT),
    ("pad slot not zero", "master[e] = 0.0f;", "master[e] = 1.0f;", LAYOUT),
    ("gather picks the wrong rank", "int64_t r = k / s;", "int64_t r = k % nd;", LAYOUT),
    ("sum starts from +0",
     "float acc = g[0];\n    for (int32_t r = 1;", "float acc = 0.0f;\n    for (int32_t r = 0;",
     REDUCE),
    ("sum in reverse rank order",
     "float acc = g[0];\n    for (int32_t r = 1; r < nd; ++r) acc = acc + g[r];",
     "float acc = g[nd - 1];\n    for (int32_t r = nd - 2; r >= 0; --r) acc = acc + g[r];",
     REDUCE),
    ("reduce reads the neighbour's slice",
     "int64_t k = (int64_t)j * s + i;          /* index in padded tensor t */",
     "int64_t k = (int64_t)((j + 1) % nd) * s + i;", REDUCE),
    ("accumulate overwrites", "acc[i] = acc[i] + g[i];", "acc[i] = g[i];", REDUCE),
    ("second moment uses 1-b1", "b2 * (*v) + omb2 * (g * g)", "b2 * (*v) + omb1 * (g * g)",
     ADAM),
    ("second moment decays with b1", "b2 * (*v) + omb2", "b1 * (*v) + omb2", ADAM),
    ("bias correction one step late", "pow((double)b1, (double)step)",
     "pow((double)b1, (double)(step + 1))", ADAM),
    ("no first-moment bias correction", "float mhat = m_new / bc1;", "float mhat = m_new;", ADAM),
    ("eps inside the square root", "sqrtf(vhat) + eps", "sqrtf(vhat + eps)", ADAM),
    ("step added instead of subtracted", "*p - update", "*p + update", ADAM),
    ("first moment never stored", "*m = m_new;", "(void)m_new;", ADAM),
    ("bf16 ties rounded down",
     "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
     "if (dropped > 0x8000u) kept += 1u;", ADAM),
    ("bf16 ties rounded away",
     "(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)", ADAM),
    ("reduce drops the last rank",
     "for (int32_t r = 1; r < nd; ++r) acc = acc + g[r];",
     "for (int32_t r = 1; r < nd - 1; ++r) acc = acc + g[r];", REDUCE),
    ("reduce reads pad slots", "if (k >= numel[t]) { out[e] = 0.0f; continue; }", "", REDUCE),
    ("gather forgets the rank's base",
     "int64_t idx = r * L.S + L.shard_off[t] + (k - r * s);",
     "int64_t idx = L.shard_off[t] + (k - r * s);", LAYOUT),
    ("shard offsets skip a slot", "shard_off[t + 1] = shard_off[t] + shard_len[t];",
     "shard_off[t + 1] = shard_off[t] + shard_len[t] + 1;", LAYOUT),
    ("bf16 cast leaves NaN unquieted",
     "return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);", ADAM),
    ("adam updates pad slots",
     "if (k >= numel[t]) continue;\n            int64_t e = L.shard_off[t] + i;\n            adam_one",
     "int64_t e = L.shard_off[t] + i;\n            adam_one", ADAM),
    # differences of one rounding, inside every bound above: the second
    # implementation (bit for bit) is what catches them
    ("update divides before scaling by lr", "float update = (lr * mhat) / denom;",
     "float update = lr * (mhat / denom);", BRUTE),
    ("g squared after scaling", "omb2 * (g * g)", "(omb2 * g) * g", BRUTE),
    ("bias correction through a reciprocal", "float mhat = m_new / bc1;",
     "float mhat = m_new * (1.0f / bc1);", BRUTE),
    ("bias corrections in fp32", "out4[2] = (float)(1.0 - pow((double)b1, (double)step));",
     "out4[2] = 1.0f - powf(b1, (float)step);", BRUTE),
]


@pytest.mark.parametrize("name,old,new,target", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, target, tmp_path):
    src = open(os.path.join(ORACLE_DIR, "oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor for '{name}' not found exactly once"
    (tmp_path / "oracle.c").write_text(src.replace(old, new))
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), tmp_path / "oracle.h")
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", *CFLAGS, "-o", str(lib), str(tmp_path / "oracle.c"), "-lm"],
                   check=True)
    env = dict(os.environ, ZSP_ORACLE_LIB=str(lib))
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", target], cwd=ROOT, env=env,
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    assert res.returncode != 0, f"pins did not catch '{name}':\n" + res.stdout.decode()[-2000:]
