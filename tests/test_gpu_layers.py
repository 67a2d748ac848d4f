"""Per-layer reduce-scatter and update: the shard calls restricted to a
parameter range ("The ZeRO-3 Diagram Most People Remember Is Wrong", §6:
gradient reduce-scatters during backward; "ZeRO Stage 3: Parameter
Partitioning": after a layer's backward its gradients are shipped to the
owning ranks). Reducing the groups one by one touches exactly their slots and
gives, bit for bit, the oracle's whole reduce; per-group updates give the
oracle's whole update."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import binding

from test_gpu_parity import CASES, HP, Mirror, assert_bits, dev, np_of

# Long pieces (two waves per tile) over several parameters whose slots start
# mid-tile, so per-group ranges cut tiles at both ends.
LONG = ([300 * 1001, 7, 200 * 513 + 3, 65536, 4096 * 9 + 1], 4)

pytestmark = pytest.mark.gpu


def groups_of(T):
    """Split T parameters into up to three consecutive, non-empty groups."""
    if T == 1:
        return [(0, 1)]
    if T == 2:
        return [(0, 1), (1, 1)]
    a, b = T // 3 or 1, (2 * T) // 3 or 2
    return [(0, a), (a, b - a), (b, T - b)]


def slot_mask(M, first, n):
    """Boolean mask over the bound state: the slots of parameters [first, first+n)."""
    L = M.L
    mask = np.zeros(M.n, bool)
    for j in M.ranks:
        base = 0 if M.rank_local is not None else j * L.S
        mask[base + int(L.shard_off[first]):base + int(L.shard_off[first + n])] = True
    return mask


@pytest.mark.parametrize("numels,nd", CASES[:9] + [LONG])
def test_reduce_by_groups(numels, nd):
    M = Mirror(numels, nd)
    grads = M.grads(torch.bfloat16, "layers-reduce")
    gdev = [g.to(dev()) for g in grads]
    M.g_acc.fill_(float("nan"))
    want = np.concatenate([M.o_reduce(j, grads) for j in M.ranks])
    written = np.zeros(M.n, bool)
    for first, n in groups_of(len(numels)):
        M.plan.reduce_shard_params(zsp.ALL_RANKS, first, n, gdev)
        torch.cuda.synchronize()
        got = np_of(M.g_acc[:M.n])
        written |= slot_mask(M, first, n)
        assert_bits(got[written], want[written], f"group [{first}, {first + n})")
        assert np.isnan(got[~written]).all(), "a slot outside the group was written"
    assert written.all()


@pytest.mark.parametrize("numels,nd", CASES[:9] + [LONG])
def test_fused_update_by_groups(numels, nd):
    M = Mirror(numels, nd)
    for step in (1, 2):
        grads = M.grads(torch.bfloat16, ("layers-fused", step))
        gdev = [g.to(dev()) for g in grads]
        for first, n in reversed(groups_of(len(numels))):   # backward order
            M.plan.reduce_adam_step_params(zsp.ALL_RANKS, first, n, gdev, step=step, **HP)
        for j in M.ranks:
            M.o_adam(j, M.o_reduce(j, grads), step)
        assert M.check_state(f"step {step}") == 0


@pytest.mark.parametrize("numels,nd", CASES[:6] + [LONG])
def test_reduce_then_adam_by_groups(numels, nd):
    M = Mirror(numels, nd)
    grads = M.grads(torch.bfloat16, "layers-acc")
    gdev = [g.to(dev()) for g in grads]
    for first, n in reversed(groups_of(len(numels))):
        M.plan.reduce_shard_params(zsp.ALL_RANKS, first, n, gdev)
    for first, n in groups_of(len(numels)):
        M.plan.adam_step_params(zsp.ALL_RANKS, first, n, step=1, **HP)
    for j in M.ranks:
        M.o_adam(j, M.o_reduce(j, grads), 1)
    assert M.check_state("reduce then adam by groups") == 0


def test_single_rank_and_rank_local_groups():
    numels, nd = [1003, 64, 5, 0, 3 * 4096 + 1, 7], 8
    M = Mirror(numels, nd)
    grads = M.grads(torch.bfloat16, "layers-one-rank")
    gdev = [g.to(dev()) for g in grads]
    M.g_acc.fill_(float("nan"))
    M.plan.reduce_shard_params(3, 1, 3, gdev)
    torch.cuda.synchronize()
    got = np_of(M.g_acc[:M.n])
    mask = np.zeros(M.n, bool)
    lo, hi = 3 * M.L.S + int(M.L.shard_off[1]), 3 * M.L.S + int(M.L.shard_off[4])
    mask[lo:hi] = True
    want = np.concatenate([M.o_reduce(j, grads) for j in M.ranks])
    assert_bits(got[mask], want[mask], "rank 3, parameters [1, 4)")
    assert np.isnan(got[~mask]).all()
    # a one-rank binding with shard-layout gradients
    R = Mirror(numels, nd, rank_local=5)
    g2 = R.grads(torch.bfloat16, "layers-local", layout="shard")
    g2dev = [g.to(dev()) for g in g2]
    for first, n in reversed(groups_of(len(numels))):
        R.plan.reduce_adam_step_params(5, first, n, g2dev, step=1, layout="shard", **HP)
    R.o_adam(5, R.o_reduce(5, g2, layout="shard"), 1)
    assert R.check_state("rank-local by groups") == 0


def test_range_errors():
    numels, nd = [1003, 64, 5], 4
    M = Mirror(numels, nd)
    gdev = [g.to(dev()) for g in M.grads(torch.bfloat16, "layers-err")]
    for first, n in ((0, 0), (-1, 1), (2, 2), (3, 1), (0, 4)):
        with pytest.raises(zsp.ZspError) as e:
            M.plan.reduce_shard_params(zsp.ALL_RANKS, first, n, gdev)
        assert e.value.status == binding.ERANGE
        with pytest.raises(zsp.ZspError) as e:
            M.plan.adam_step_params(zsp.ALL_RANKS, first, n, step=1, **HP)
        assert e.value.status == binding.ERANGE
    with pytest.raises(zsp.ZspError) as e:
        M.plan.reduce_shard_params(4, 0, 1, gdev)
    assert e.value.status == binding.EINVAL
