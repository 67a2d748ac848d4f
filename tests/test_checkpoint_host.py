"""Sharded checkpoint files on the host (no GPU): per-rank write/read round
trip, resharding to another rank count, and rejection of damaged or foreign
files ("ZeRO Stages: Sharding Optimizer State, Gradients, and Parameters",
"Where the shards live and what happens on failure").

Expected shards come from the oracle: gather every parameter out of the old
rank count's shards, then partition it under the new one.
"""
import os

import numpy as np
import pytest
import xxhash

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import binding


def state_for(numels, nd, seed):
    """All ranks' master/m/v/work as the oracle lays them out, with m and v
    holding nonzero values so that every array is checked."""
    L = oracle.Layout(numels, nd)
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(L.total_numel) * 0.02).astype(np.float32)
    master, work, _, _ = oracle.partition(numels, nd, x)
    m_flat = (rng.standard_normal(L.total_numel) * 1e-3).astype(np.float32)
    v_flat = (rng.random(L.total_numel) * 1e-6).astype(np.float32)
    m, _, _, _ = oracle.partition(numels, nd, m_flat)
    v, _, _, _ = oracle.partition(numels, nd, v_flat)
    return L, master, m, v, work


def gathered(numels, nd, arr):
    return np.concatenate([oracle.gather(numels, nd, t, arr) for t in range(len(numels))])


def write_all(plan, d, L, master, m, v, work, step):
    for r in range(L.nd):
        sl = slice(r * L.S, (r + 1) * L.S)
        plan.checkpoint_write_host(r, d, step, master[sl], m[sl], v[sl], work[sl])


def check_file(path, numels, nd, r, S, step, arrays):
    """The file's bytes are the documented layout, and its trailing checksum
    is XXH64 (seed 0) of everything before it, as the xxhash package computes."""
    raw = open(path, "rb").read()
    want = (b"ZSPCKPT1" + np.array([nd, r, len(numels), S, step], "<i8").tobytes()
            + np.array(numels, "<i8").tobytes()
            + b"".join(np.ascontiguousarray(a).tobytes() for a in arrays))
    assert raw[:-8] == want
    assert int.from_bytes(raw[-8:], "little") == xxhash.xxh64(want, seed=0).intdigest()


def read_rank(plan, d, S, r):
    out = [np.empty(S, np.float32) for _ in range(3)] + [np.empty(S, np.uint16)]
    step = plan.checkpoint_read_host(r, d, *out)
    return step, out


CASES = [([1003, 64, 5, 0, 3 * 4096 + 1], 8), ([97, 0, 12345], 4), ([7] * 20 + [1000], 16),
         ([1000 * 1003], 4), ([1, 2, 3], 1)]


@pytest.mark.parametrize("numels,nd", CASES)
def test_roundtrip_same_layout(tmp_path, numels, nd):
    L, master, m, v, work = state_for(numels, nd, 0)
    plan = zsp.partition(numels, nd)
    write_all(plan, str(tmp_path), L, master, m, v, work, step=42)
    assert sorted(os.listdir(tmp_path)) == sorted(f"rank-{r}-of-{nd}.zsp" for r in range(nd))
    for r in range(nd):
        check_file(os.path.join(tmp_path, f"rank-{r}-of-{nd}.zsp"), numels, nd, r, L.S, 42,
                   [a[r * L.S:(r + 1) * L.S] for a in (master, m, v, work)])
    for r in range(nd):
        step, (a, b, c, d) = read_rank(plan, str(tmp_path), L.S, r)
        sl = slice(r * L.S, (r + 1) * L.S)
        assert step == 42
        for got, want in ((a, master), (b, m), (c, v), (d, work)):
            assert np.array_equal(got.view(np.uint8), want[sl].view(np.uint8))
    plan.destroy()


RESHARD = [(8, 4), (4, 8), (3, 5), (8, 1), (1, 7), (16, 3), (5, 5)]


@pytest.mark.parametrize("nd_old,nd_new", RESHARD)
def test_reshard_matches_gather_then_partition(tmp_path, nd_old, nd_new):
    numels = [1003, 64, 5, 0, 3 * 4096 + 1, 7, 1]
    Lo, master, m, v, work = state_for(numels, nd_old, 1)
    old = zsp.partition(numels, nd_old)
    write_all(old, str(tmp_path), Lo, master, m, v, work, step=7)
    Ln = oracle.Layout(numels, nd_new)
    want_master, _, _, _ = oracle.partition(numels, nd_new, gathered(numels, nd_old, master))
    want_m, _, _, _ = oracle.partition(numels, nd_new, gathered(numels, nd_old, m))
    want_v, _, _, _ = oracle.partition(numels, nd_new, gathered(numels, nd_old, v))
    _, want_work, _, _ = oracle.partition(numels, nd_new, gathered(numels, nd_old, work))
    new = zsp.partition(numels, nd_new)
    for r in range(nd_new):
        step, got = read_rank(new, str(tmp_path), Ln.S, r)
        sl = slice(r * Ln.S, (r + 1) * Ln.S)
        assert step == 7
        for g, w in zip(got, (want_master, want_m, want_v, want_work)):
            assert np.array_equal(g.view(np.uint8), w[sl].view(np.uint8))
    old.destroy()
    new.destroy()


def _status(fn, *args):
    try:
        fn(*args)
    except zsp.ZspError as e:
        return e.status
    return 0


def test_damaged_and_foreign_files_are_rejected(tmp_path):
    numels, nd = [1003, 64, 5], 4
    L, master, m, v, work = state_for(numels, nd, 2)
    plan = zsp.partition(numels, nd)
    d = str(tmp_path)
    out = [np.empty(L.S, np.float32) for _ in range(3)] + [np.empty(L.S, np.uint16)]
    assert _status(plan.checkpoint_read_host, 0, d, *out) == binding.EIO   # empty dir
    write_all(plan, d, L, master, m, v, work, step=1)
    path = os.path.join(d, "rank-2-of-4.zsp")
    good = open(path, "rb").read()
    # a flipped payload byte fails the hash
    bad = bytearray(good)
    bad[len(bad) // 2] ^= 0x40
    open(path, "wb").write(bytes(bad))
    assert _status(plan.checkpoint_read_host, 2, d, *out) == binding.EIO
    assert "corrupt" in zsp.last_error()
    # a truncated file
    open(path, "wb").write(good[:-9])
    assert _status(plan.checkpoint_read_host, 2, d, *out) == binding.EIO
    # a trailing extra byte
    open(path, "wb").write(good + b"\0")
    assert _status(plan.checkpoint_read_host, 2, d, *out) == binding.EIO
    open(path, "wb").write(good)
    assert _status(plan.checkpoint_read_host, 2, d, *out) == 0
    # another model's parameter list, with the same S and with a larger one
    other = zsp.partition([1003, 64, 6], nd)
    assert _status(other.checkpoint_read_host, 0, d, *out) == binding.EIO
    assert "another parameter list" in zsp.last_error()
    small = zsp.partition([1003], nd)
    Ls = oracle.Layout([1003], nd)
    outs = [np.zeros(Ls.S, np.float32) for _ in range(3)] + [np.zeros(Ls.S, np.uint16)]
    assert _status(small.checkpoint_read_host, 0, d, *outs) == binding.EIO
    assert "another parameter list" in zsp.last_error()
    assert all(not a.any() for a in outs)   # refused before any payload was written
    small.destroy()
    # resharding needs every old rank file, all at one step
    eight = zsp.partition(numels, 8)
    L8 = oracle.Layout(numels, 8)
    out8 = [np.empty(L8.S, np.float32) for _ in range(3)] + [np.empty(L8.S, np.uint16)]
    os.rename(path, path + ".away")
    assert _status(eight.checkpoint_read_host, 0, d, *out8) == binding.EIO
    os.rename(path + ".away", path)
    sl = slice(2 * L.S, 3 * L.S)
    plan.checkpoint_write_host(2, d, 5, master[sl], m[sl], v[sl], work[sl])
    assert _status(eight.checkpoint_read_host, 0, d, *out8) == binding.EIO
    assert "mixes steps" in zsp.last_error()
    # argument errors
    assert _status(plan.checkpoint_read_host, 4, d, *out) == binding.EINVAL
    with pytest.raises(TypeError):
        plan.checkpoint_write_host(0, d, 1, master[:L.S].astype(np.float64), m, v, work)
    for p in (plan, other, eight):
        p.destroy()


def test_no_temporary_files_left(tmp_path):
    numels, nd = [300, 17], 3
    L, master, m, v, work = state_for(numels, nd, 3)
    plan = zsp.partition(numels, nd)
    write_all(plan, str(tmp_path), L, master, m, v, work, step=9)
    write_all(plan, str(tmp_path), L, master, m, v, work, step=10)   # overwrite
    assert not [f for f in os.listdir(tmp_path) if f.endswith(".tmp")]
    assert read_rank(plan, str(tmp_path), L.S, 1)[0] == 10
    plan.destroy()


def test_single_rank_file_and_mixed_rank_counts(tmp_path):
    numels, nd = [1003, 64, 5], 4
    L, master, m, v, work = state_for(numels, nd, 4)
    plan = zsp.partition(numels, nd)
    d = str(tmp_path)
    sl = slice(3 * L.S, 4 * L.S)
    plan.checkpoint_write_host(3, d, 11, master[sl], m[sl], v[sl], work[sl])
    step, got = read_rank(plan, d, L.S, 3)          # only rank 3's file exists
    assert step == 11
    assert np.array_equal(got[0].view(np.uint32), master[sl].view(np.uint32))
    out = [np.empty(L.S, np.float32) for _ in range(3)] + [np.empty(L.S, np.uint16)]
    assert _status(plan.checkpoint_read_host, 0, d, *out) == binding.EIO
    other = zsp.partition(numels, 2)
    L2 = oracle.Layout(numels, 2)
    other.checkpoint_write_host(0, d, 11, *[a[:L2.S] for a in (master, m, v, work)])
    assert _status(plan.checkpoint_read_host, 3, d, *out) == binding.EIO
    assert "several rank counts" in zsp.last_error()
    plan.destroy()
    other.destroy()
