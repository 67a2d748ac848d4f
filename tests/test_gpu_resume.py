"""Elastic resume: train at one rank count, save a sharded checkpoint, load
it under another rank count and keep training ("ZeRO Stages: Sharding
Optimizer State, Gradients, and Parameters", "Where the shards live and what
happens on failure": a restart under another rank count reshuffles the
shards). The oracle follows the same path: its state, viewed in the
unpadded parameter order, does not depend on the rank count, so it is
resharded by gathering it under the old count and partitioning it under the
new one. Every step's state must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle

from test_gpu_parity import HP, Mirror, dev

pytestmark = pytest.mark.gpu

NUMELS = [1003, 64, 5, 0, 3 * 4096 + 1, 4096 * 2 + 7, 17]


def flat_of(numels, nd, arr):
    """The unpadded concatenation of every parameter of an all-rank array."""
    parts = [oracle.gather(numels, nd, t, arr) for t in range(len(numels))]
    return np.concatenate(parts) if parts else arr[:0]


def reshard(numels, nd_old, nd_new, master, m, v, work):
    """The oracle's state under nd_new: each array gathered under nd_old and
    partitioned under nd_new (the partition's pads are +0, like the state's)."""
    out = []
    for arr in (master, m, v):
        new_master, _w, _m, _v = oracle.partition(numels, nd_new, flat_of(numels, nd_old, arr))
        out.append(new_master)
    _m2, new_work, _m3, _v3 = oracle.partition(numels, nd_new, flat_of(numels, nd_old, work))
    out.append(new_work)
    return out


def train(M, first_step, n_steps, tag):
    for step in range(first_step, first_step + n_steps):
        grads = M.grads(torch.bfloat16, f"{tag}-{step}")
        M.plan.reduce_adam_step(-1, [g.to(dev()) for g in grads], step=step, **HP)
        for j in range(M.nd):
            M.o_adam(j, M.o_reduce(j, grads), step)
        M.check_state(f"{tag} step {step}", exact=True)


@pytest.mark.parametrize("nd_old,nd_new", [(8, 4), (3, 7)])
def test_train_save_reshard_resume(nd_old, nd_new, tmp_path):
    A = Mirror(NUMELS, nd_old, seed=1)
    train(A, 1, 2, f"before n_d={nd_old}")
    A.plan.checkpoint_save(-1, str(tmp_path), step=2)
    torch.cuda.synchronize()

    B = Mirror(NUMELS, nd_new, seed=2)  # other initial values, overwritten by the load
    assert B.plan.checkpoint_load(-1, str(tmp_path)) == 2
    B.o_master[:], B.o_m[:], B.o_v[:], B.o_work[:] = reshard(
        NUMELS, nd_old, nd_new, A.o_master, A.o_m, A.o_v, A.o_work)
    B.check_state(f"loaded under n_d={nd_new}", exact=True)
    train(B, 3, 2, f"after n_d={nd_new}")
