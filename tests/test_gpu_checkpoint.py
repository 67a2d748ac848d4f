"""Sharded checkpoint through the device entry points: save between steps,
lose state, load, continue -- bit-identical to an uninterrupted run; restore
one lost virtual rank alone; load under another rank count (reshard)."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp

from test_gpu_parity import HP, Mirror, assert_bits, np_of

pytestmark = pytest.mark.gpu

NUMELS = [1003, 64, 5, 0, 3 * 4096 + 1, 7]


def state_bits(M):
    torch.cuda.synchronize()
    return [np_of(x[:M.n]) for x in (M.g_master, M.g_m, M.g_v, M.g_work)]


def step(M, grads, t, layout="full"):
    M.plan.reduce_adam_step(zsp.ALL_RANKS if M.rank_local is None else M.rank_local,
                            [g.to("cuda") for g in grads], step=t, layout=layout, **HP)


def test_resume_is_bit_identical(tmp_path):
    nd = 4
    A, B = Mirror(NUMELS, nd), Mirror(NUMELS, nd)
    grads = [A.grads(torch.bfloat16, ("ckpt", t)) for t in range(1, 5)]
    for t in (1, 2):
        step(A, grads[t - 1], t)
        step(B, grads[t - 1], t)
    A.plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 2)
    for x in (A.g_master, A.g_m, A.g_v):
        x.fill_(float("nan"))
    A.g_work.fill_(3.0)
    assert A.plan.checkpoint_load(zsp.ALL_RANKS, str(tmp_path)) == 2
    for got, want in zip(state_bits(A), state_bits(B)):
        assert_bits(got, want, "state after load")
    for t in (3, 4):
        step(A, grads[t - 1], t)
        step(B, grads[t - 1], t)
    for got, want, name in zip(state_bits(A), state_bits(B), ("master", "m", "v", "work")):
        assert_bits(got, want, f"after resume: {name}")


def test_restore_one_lost_rank(tmp_path):
    nd = 8
    A = Mirror(NUMELS, nd)
    step(A, A.grads(torch.bfloat16, "lost"), 1)
    before = state_bits(A)
    A.plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 1)
    lost = 5
    sl = slice(lost * A.L.S, (lost + 1) * A.L.S)
    for x in (A.g_master, A.g_m, A.g_v):
        x[sl].fill_(0.0)
    A.g_work[sl].fill_(0.0)
    assert A.plan.checkpoint_load(lost, str(tmp_path)) == 1
    for got, want, name in zip(state_bits(A), before, ("master", "m", "v", "work")):
        assert_bits(got, want, f"rank {lost} restored: {name}")


@pytest.mark.parametrize("nd_old,nd_new", [(8, 4), (4, 8), (3, 5)])
def test_load_reshards(tmp_path, nd_old, nd_new):
    A = Mirror(NUMELS, nd_old)
    step(A, A.grads(torch.bfloat16, "reshard"), 1)
    old = state_bits(A)
    A.plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 1)
    B = Mirror(NUMELS, nd_new)
    assert B.plan.checkpoint_load(zsp.ALL_RANKS, str(tmp_path)) == 1
    got = state_bits(B)

    def regathered(arr):
        return np.concatenate([oracle.gather(NUMELS, nd_old, t, arr) for t in range(len(NUMELS))])

    want_master, _, _, _ = oracle.partition(NUMELS, nd_new, regathered(old[0]))
    want_m, _, _, _ = oracle.partition(NUMELS, nd_new, regathered(old[1]))
    want_v, _, _, _ = oracle.partition(NUMELS, nd_new, regathered(old[2]))
    _, want_work, _, _ = oracle.partition(NUMELS, nd_new, regathered(old[3]))
    for g, w, name in zip(got, (want_master, want_m, want_v, want_work),
                          ("master", "m", "v", "work")):
        assert_bits(g, w, f"resharded {nd_old}->{nd_new}: {name}")
    # the resharded state gathers back to the same parameters
    out = torch.empty(B.L.total_numel, dtype=torch.float32, device="cuda")
    B.plan.gather_range(0, len(NUMELS), out, "master")
    torch.cuda.synchronize()
    assert_bits(np_of(out), regathered(old[0]), "gather after reshard")


def test_rank_local_binding(tmp_path):
    nd, j = 16, 6
    A = Mirror(NUMELS, nd, rank_local=j)
    step(A, A.grads(torch.bfloat16, "local", layout="shard"), 1, layout="shard")
    step(A, A.grads(torch.bfloat16, "local2", layout="shard"), 2, layout="shard")
    before = state_bits(A)
    A.plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 2)
    assert sorted(p.name for p in tmp_path.iterdir()) == [f"rank-{j}-of-{nd}.zsp"]
    for x in (A.g_master, A.g_m, A.g_v):
        x.fill_(1.0)
    assert A.plan.checkpoint_load(j, str(tmp_path)) == 2
    for got, want in zip(state_bits(A), before):
        assert_bits(got, want, "rank-local restore")
    with pytest.raises(zsp.ZspError) as e:
        A.plan.checkpoint_load((j + 1) % nd, str(tmp_path))
    assert e.value.status == zsp.binding.ESTATE


def test_state_spanning_many_chunks(tmp_path):
    """Each state array larger than one 16 MiB staging chunk (S = 6.5M), and
    two ranks' files written and read in parallel."""
    numels = [9_000_001, 4_000_003, 77]
    A, B = Mirror(numels, 2, with_acc=False), Mirror(numels, 2, with_acc=False)
    grads = A.grads(torch.bfloat16, "big", poison=False)
    step(A, grads, 1)
    step(B, grads, 1)
    A.plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 1)
    for x in (A.g_master, A.g_m, A.g_v):
        x.fill_(float("nan"))
    A.g_work.fill_(7.0)
    assert A.plan.checkpoint_load(zsp.ALL_RANKS, str(tmp_path)) == 1
    for got, want, name in zip(state_bits(A), state_bits(B), ("master", "m", "v", "work")):
        assert_bits(got, want, f"many chunks: {name}")


def test_more_ranks_than_lanes_and_stream_order(tmp_path):
    """Twelve rank files over fewer worker lanes; the save is queued right
    after a step on a non-blocking stream, with no host wait in between, and
    must hold the state after that step."""
    nd = 12
    A, B = Mirror(NUMELS, nd), Mirror(NUMELS, nd)
    g1 = A.grads(torch.bfloat16, "lanes1")
    g2 = A.grads(torch.bfloat16, "lanes2")
    step(A, g1, 1)
    step(B, g1, 1)
    step(B, g2, 2)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    gdev = [g.to("cuda") for g in g2]
    torch.cuda.synchronize()
    A.plan.reduce_adam_step(zsp.ALL_RANKS, gdev, step=2, stream=s, **HP)
    A.plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 2, stream=s)
    assert len(list(tmp_path.iterdir())) == nd
    C = Mirror(NUMELS, nd)
    torch.cuda.synchronize()   # C's copy-in ran on the default stream
    assert C.plan.checkpoint_load(zsp.ALL_RANKS, str(tmp_path), stream=s) == 2
    for got, want, name in zip(state_bits(C), state_bits(B), ("master", "m", "v", "work")):
        assert_bits(got, want, f"saved after the queued step: {name}")


def test_reshard_of_a_state_spanning_many_chunks(tmp_path):
    """Saved by 2 ranks, loaded by 3: each new array (S = 4.33M) spans more
    than one 16 MiB staging chunk, so chunk windows split parameters."""
    numels = [9_000_001, 4_000_003, 77]
    A = Mirror(numels, 2, with_acc=False)
    step(A, A.grads(torch.bfloat16, "big-reshard", poison=False), 1)
    old = state_bits(A)
    A.plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 1)
    B = Mirror(numels, 3, with_acc=False)
    torch.cuda.synchronize()
    assert B.plan.checkpoint_load(zsp.ALL_RANKS, str(tmp_path)) == 1
    got = state_bits(B)

    def regathered(arr):
        return np.concatenate([oracle.gather(numels, 2, t, arr) for t in range(len(numels))])

    want_master, _, _, _ = oracle.partition(numels, 3, regathered(old[0]))
    want_m, _, _, _ = oracle.partition(numels, 3, regathered(old[1]))
    want_v, _, _, _ = oracle.partition(numels, 3, regathered(old[2]))
    _, want_work, _, _ = oracle.partition(numels, 3, regathered(old[3]))
    for g, w, name in zip(got, (want_master, want_m, want_v, want_work),
                          ("master", "m", "v", "work")):
        assert_bits(g, w, f"resharded 2->3, many chunks: {name}")
