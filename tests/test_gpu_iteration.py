"""One stage-3 iteration composed from the library's calls, as a runtime
would run it ("ZeRO Stage 3: Parameter Partitioning", on-demand fetch list;
"The ZeRO-3 Diagram Most People Remember Is Wrong", §6): layers gathered
through the schedule (depth 1) for forward and backward, each layer's
gradients reduced into the accumulator during backward, then one Adam step.
The state must equal, bit for bit, that of the single fused call on the same
gradients, and every gathered layer must equal the oracle's gather."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp

from test_gpu_parity import HP, Mirror, assert_bits, dev, np_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nd", [8, 3])
def test_iteration_equals_fused_step(nd):
    layer = [1003, 64, 5, 2048, 7]
    L = 4
    numels = layer * L
    A = Mirror(numels, nd)          # composed iteration
    B = Mirror(numels, nd)          # the fused call
    groups = [(len(layer) * l, len(layer)) for l in range(L)]
    order = list(range(L)) + list(reversed(range(L)))
    sched = zsp.Schedule(A.plan, groups, order, depth=1)
    arena = torch.empty(sched.arena_bytes, dtype=torch.uint8, device=dev())
    cs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    sched.bind(arena, gs)
    torch.cuda.synchronize()
    for step in (1, 2):
        grads = A.grads(torch.bfloat16, ("iteration", step))
        gdev = [g.to(dev()) for g in grads]
        torch.cuda.synchronize()
        seen = []
        with torch.cuda.stream(cs):
            for p, l in enumerate(order):
                views = sched.acquire(p, cs)
                seen.append([v.clone() for v in views])       # the "compute"
                sched.release(p, cs)
                if p >= L:
                    A.plan.reduce_shard_params(zsp.ALL_RANKS, *groups[l], gdev, stream=cs)
            A.plan.adam_step(zsp.ALL_RANKS, step=step, stream=cs, **HP)
        B.plan.reduce_adam_step(zsp.ALL_RANKS, gdev, step=step, **HP)
        torch.cuda.synchronize()
        for p, l in enumerate(order):
            f, c = groups[l]
            for i, t in enumerate(range(f, f + c)):
                assert_bits(np_of(seen[p][i]), oracle.gather(numels, nd, t, B.o_work),
                            f"step {step} position {p} parameter {t}")
        for name, a, b in (("master", A.g_master, B.g_master), ("m", A.g_m, B.g_m),
                           ("v", A.g_v, B.g_v), ("work", A.g_work, B.g_work)):
            assert_bits(np_of(a[:A.n]), np_of(b[:B.n]), f"step {step} {name}")
        for j in range(nd):
            B.o_adam(j, B.o_reduce(j, grads), step)
        assert B.check_state(f"step {step}") == 0
    sched.destroy()
