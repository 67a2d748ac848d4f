"""Several host threads on one plan, each acting on its own rank: the
reduce + Adam + cast and the gather calls only read the plan, so one thread
per rank, each on its own stream, gives the oracle's result bit for bit
("ZeRO Stage 3: Parameter Partitioning": each rank reduces into and updates
only the shard it owns)."""
import threading

import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp

from test_gpu_parity import HP, Mirror, assert_bits, dev, np_of

pytestmark = pytest.mark.gpu

NUMELS = [4096 * 257 + 3, 17, 1000 * 1003, 65536 * 3, 5, 0, 4095]


def run_threads(n, fn):
    errors = []
    barrier = threading.Barrier(n)

    def body(i):
        try:
            barrier.wait()
            fn(i)
        except BaseException as e:  # reported in the main thread
            errors.append((i, e))

    threads = [threading.Thread(target=body, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors


@pytest.mark.parametrize("nd", [8, 5])
def test_one_thread_per_rank(nd):
    M = Mirror(NUMELS, nd)
    steps = 3
    grads = [M.grads(torch.bfloat16, f"threads-{s}") for s in range(steps)]
    gdev = [[g.to(dev()) for g in gs] for gs in grads]
    torch.cuda.synchronize()

    def rank_steps(j):
        s = torch.cuda.Stream()
        for step in range(1, steps + 1):
            M.plan.reduce_adam_step(j, gdev[step - 1], step=step, stream=s, **HP)
        s.synchronize()

    run_threads(nd, rank_steps)
    for step in range(1, steps + 1):
        for j in range(nd):
            M.o_adam(j, M.o_reduce(j, grads[step - 1]), step)
    M.check_state(f"{nd} threads, {steps} steps", exact=True)


def test_threads_gathering_different_parameters():
    M = Mirror(NUMELS, 8)
    L = oracle.Layout(NUMELS, 8)
    outs = [torch.empty(max(n, 1), dtype=torch.bfloat16, device=dev()) for n in NUMELS]
    torch.cuda.synchronize()

    def gather(t):
        s = torch.cuda.Stream()
        for _ in range(4):
            M.plan.gather(t, outs[t][:NUMELS[t]], "work", stream=s)
        s.synchronize()

    run_threads(len(NUMELS), gather)
    for t, n in enumerate(NUMELS):
        assert_bits(np_of(outs[t][:n]), oracle.gather(NUMELS, 8, t, M.o_work), f"parameter {t}")
