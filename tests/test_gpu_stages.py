"""ZeRO stage 1 and 2 step schedules from the same kernels ("ZeRO Stages:
Sharding Optimizer State, Gradients, and Parameters", stage 1 and stage 2
sections), against the oracle and against the stage-3 path:
  stage 1: reduce-scatter into the accumulator, all-gather of it (the
           all-reduced gradient every rank holds), Adam from each rank's
           slice, then each rank's new slice gathered into the full copy;
  stage 2: fused reduce-scatter + Adam, one all-gather of the parameters;
  stage 3: fused reduce-scatter + Adam (per-layer gathers happen around
           compute, not here).
The update is the same arithmetic in every stage, so the states agree bit for
bit."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import binding

from test_gpu_parity import CASES, HP, Mirror, assert_bits, dev, np_of

pytestmark = pytest.mark.gpu


def o_allreduced(M, grads):
    """The oracle's reduced slices of every rank, gathered per parameter:
    the full gradient sum a stage-1 all-reduce leaves on every rank."""
    red = np.concatenate([M.o_reduce(j, grads) for j in range(M.nd)])
    return np.concatenate([oracle.gather(M.numels, M.nd, t, red) for t in range(M.L.T)]), red


@pytest.mark.parametrize("numels,nd", CASES[:8])
def test_acc_gather_is_the_allreduced_gradient(numels, nd):
    M = Mirror(numels, nd)
    grads = M.grads(torch.bfloat16, "stage1-ar")
    gdev = [g.to(dev()) for g in grads]
    M.plan.reduce_shard(zsp.ALL_RANKS, gdev, accumulate=False)
    out = torch.empty(max(M.L.total_numel, 1), dtype=torch.float32, device=dev())
    M.plan.gather_range(0, M.L.T, out[:M.L.total_numel], "acc")
    torch.cuda.synchronize()
    want, red = o_allreduced(M, grads)
    assert_bits(np_of(M.g_acc[:M.n]), red, "reduced slices")
    assert_bits(np_of(out[:M.L.total_numel]), want.astype(np.float32), "all-reduced gradient")
    # one parameter at a time gives the same values
    k = 0
    for t in range(M.L.T):
        n = M.numels[t]
        if n:
            o = torch.empty(n, dtype=torch.float32, device=dev())
            M.plan.gather(t, o, "acc")
            torch.cuda.synchronize()
            assert_bits(np_of(o), want[k:k + n].astype(np.float32), f"parameter {t}")
        k += n


def run_stage(M, stage, grads, step):
    gdev = [g.to(dev()) for g in grads]
    p = M.plan
    full = torch.empty(max(M.L.total_numel, 1), dtype=torch.bfloat16, device=dev())
    if stage == 1:
        replica = torch.empty(max(M.L.total_numel, 1), dtype=torch.float32, device=dev())
        p.reduce_shard(zsp.ALL_RANKS, gdev, accumulate=False)
        p.gather_range(0, M.L.T, replica[:M.L.total_numel], "acc")
        p.adam_step(zsp.ALL_RANKS, step=step, **HP)
    else:
        p.reduce_adam_step(zsp.ALL_RANKS, gdev, step=step, **HP)
    p.gather_range(0, M.L.T, full[:M.L.total_numel], "work")
    torch.cuda.synchronize()
    return np_of(full[:M.L.total_numel])


@pytest.mark.parametrize("numels,nd", CASES[:8])
def test_stage_schedules_agree_with_each_other_and_the_oracle(numels, nd):
    mirrors = {s: Mirror(numels, nd) for s in (1, 2, 3)}
    O = mirrors[3]
    for step in (1, 2):
        grads = O.grads(torch.bfloat16, ("stages", step))
        replicas = {s: run_stage(M, s, grads, step) for s, M in mirrors.items()}
        for j in range(nd):
            O.o_adam(j, O.o_reduce(j, grads), step)
        want_rep = np.concatenate([oracle.gather(numels, nd, t, O.o_work)
                                   for t in range(O.L.T)]).astype(np.uint16)
        for s, M in mirrors.items():
            torch.cuda.synchronize()
            for name, x, w in (("master", M.g_master, O.o_master), ("m", M.g_m, O.o_m),
                               ("v", M.g_v, O.o_v), ("work", M.g_work, O.o_work)):
                assert_bits(np_of(x[:M.n]), w, f"stage {s} step {step} {name}")
            assert_bits(replicas[s], want_rep, f"stage {s} step {step} parameter replica")


def test_acc_gather_needs_an_accumulator():
    M = Mirror([1003, 64], 4, with_acc=False)
    out = torch.empty(1067, dtype=torch.float32, device=dev())
    with pytest.raises(zsp.ZspError) as e:
        M.plan.gather_range(0, 2, out, "acc")
    assert e.value.status == binding.ESTATE
    with pytest.raises(TypeError):
        M.plan.gather_range(0, 2, out.to(torch.bfloat16), "acc")   # fp32 only
