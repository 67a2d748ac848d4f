"""The library's offset tables satisfy every property its kernels index by
(CPU only): pieces ordered and non-empty, every gradient / parameter /
gather source range inside its buffer, each tile-table entry naming the
piece that holds the tile's first element, the gather's per-tile deltas
and two-piece records matching a search of the piece starts, and the span
gather's records, whose addressing (runs into LDS, then each element's
piece offset, found as the kernel finds it) is emulated for every element.
Built from the library's own host code with g++ (AddressSanitizer and UBSan
on) and driven over small edge cases, seeded random layouts and the full
workloads."""
import os
import subprocess

import numpy as np
import pytest

from zero_sharded_mixed_pad_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_mixed_pad_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("tables") / "table_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(ROOT, "tests", "table_check.cpp"),
                    os.path.join(CSRC, "zsp_layout.cpp"), "-o", exe], check=True)
    return exe


def run(exe, numels, nd, rank, force_spans=False):
    """Check the tables of one layout; returns the number of spans."""
    inp = f"{nd} {rank} {len(numels)} " + " ".join(str(n) for n in numels)
    if force_spans:
        inp += " 1"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    res = subprocess.run([exe], input=inp.encode(), stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, timeout=600, env=env)
    out = res.stdout.decode()
    assert res.returncode == 0 and out.startswith("ok"), out
    return int(out.split()[3])


SMALL = [
    ([1003, 64, 5, 0, 3 * 4096 + 1], 4), ([0], 4), ([0, 0, 3], 8), ([1], 1), ([1], 256),
    ([511 * 8, 512 * 8, 513 * 8], 8), ([7] * 300, 64), ([1000 * 1003], 4), ([1001 * 1003], 4),
    (synth.small_tensor_sizes(count=500, lo=1, hi=5000, seed=3), 8),
]


@pytest.mark.parametrize("numels,nd", SMALL)
def test_small_tables(checker, numels, nd):
    for rank in [-1, 0, nd - 1, nd // 2]:
        run(checker, numels, nd, rank, force_spans=True)


def test_span_tables_where_the_span_gather_runs(checker):
    """The 10,000-tensor workload and the layouts of the GPU span-gather tests
    get span tables (the gather's span form runs on them), every span
    emulated as the kernel addresses it; layouts where one tile meets more
    ranks than a span record holds get none and gather by tiles."""
    w = synth.workloads()["small_tensors_10k_nd8"]
    assert run(checker, w.numel, w.n_d, -1) > 0
    import test_gpu_span_gather as sg
    for name, (numels, nd) in sg.LAYOUTS.items():
        spans = run(checker, numels, nd, -1)
        assert (spans > 0) == (name not in sg.TILE_FORM), name


@pytest.mark.parametrize("name", list(synth.workloads()))
def test_workload_tables(checker, name):
    w = synth.workloads()[name]
    run(checker, w.numel, w.n_d, -1 if w.rank_local < 0 else w.rank_local)
    if w.rank_local < 0:
        run(checker, w.numel, w.n_d, w.n_d - 1)


def test_decoder_stack_tables(checker):
    """The 32-layer stack the gather schedule walks: 6.48e9 state elements,
    beyond 32-bit indexing in every table."""
    w = synth.llama_stack(32, 8)
    assert sum(w.numel) > 2 ** 32
    run(checker, w.numel, w.n_d, -1)


@pytest.mark.parametrize("seed", range(6))
def test_random_layout_tables(checker, seed):
    """Seeded random layouts: parameter sizes spread over five decades (zero
    included), so tiles hold one, two or many pieces and slices start at
    every alignment. Seed s takes the rank counts 12s+1 .. 12s+12, so the six
    seeds cover every rank count from 1 to 70, each with its own layout."""
    rng = np.random.default_rng(1000 + seed)
    for nd in range(12 * seed + 1, min(12 * seed + 13, 71)):
        count = int(rng.integers(1, 120))
        numels = [int(x) for x in np.floor(np.exp(rng.uniform(0, np.log(2e5), count)))]
        numels = [0 if rng.random() < 0.05 else n for n in numels]
        for rank in (-1, int(rng.integers(0, nd))):
            run(checker, numels, nd, rank, force_spans=True)
