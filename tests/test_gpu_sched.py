"""Per-layer gather schedule with prefetch on the GPU: every position's
gathered group, as the compute stream sees it right after acquire, equals the
oracle's gather of that layer ("ZeRO Stage 3: Parameter Partitioning",
on-demand fetch list and prefetch paragraph; "ZeRO Stages: ...", "Stage 3
partitions parameters"). The compute stand-in is made slow (so that a gather
overwriting a slot still in use would land inside the window) or trivial (so
that compute reading a slot before its gather finished would show); a second
pass after an Adam step on the compute stream must see the updated weights."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import binding

from test_gpu_parity import HP, Mirror, assert_bits, dev, np_of

pytestmark = pytest.mark.gpu

# six "layers", three or four parameters each, padded and unpadded, one empty
LAYERS = [[4096 * 257 + 3, 17, 4096, 1003], [65536 * 9, 5, 0], [1000 * 1003, 64, 777],
          [8 * 40000, 4096 * 11, 1, 2], [3 * 4096 + 1, 250000, 33], [524288 * 3, 9, 4095]]


def model():
    numels, groups = [], []
    for layer in LAYERS:
        groups.append((len(numels), len(layer)))
        numels += layer
    return numels, groups


def fwd_bwd(n):
    return list(range(n)) + list(range(n - 1, -1, -1))


def expected(M, groups, order, src="work"):
    arr = M.o_work if src == "work" else M.o_master
    out = []
    for g in order:
        f, c = groups[g]
        out.append([oracle.gather(M.numels, M.nd, t, arr) for t in range(f, f + c)])
    return out


def run_pass(sched, cs, slow, delay):
    """One pass over the schedule on compute stream `cs`; returns, per
    position, copies of the group's parameters taken on the compute stream."""
    caps = []
    with torch.cuda.stream(cs):
        for p in range(len(sched.order)):
            views = sched.acquire(p, cs)
            if slow:
                for _ in range(3):
                    torch.mm(delay, delay)
            caps.append([v.clone() for v in views])
            sched.release(p, cs)
    return caps


def check(caps, want, what):
    torch.cuda.synchronize()
    for p, (got_p, want_p) in enumerate(zip(caps, want)):
        for i, (g, w) in enumerate(zip(got_p, want_p)):
            assert_bits(np_of(g), w, f"{what}: position {p}, parameter {i}")


@pytest.mark.parametrize("depth", [0, 1, 2, 5])
@pytest.mark.parametrize("slow", [True, False])
@pytest.mark.parametrize("nd", [8, 3])
def test_every_position_sees_its_layer(depth, slow, nd):
    numels, groups = model()
    M = Mirror(numels, nd, with_acc=False)
    order = fwd_bwd(len(groups))
    s = zsp.Schedule(M.plan, groups, order, depth)
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=dev())
    cs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    s.bind(arena, gs if depth > 0 else None)
    torch.cuda.synchronize()
    delay = torch.randn(2048, 2048, device=dev(), dtype=torch.bfloat16)
    want = expected(M, groups, order)
    for rep in range(2):  # a second pass over the same state reuses the slots
        caps = run_pass(s, cs, slow, delay)
        check(caps, want, f"depth {depth} slow {slow} pass {rep}")
    s.destroy()


@pytest.mark.parametrize("depth", [0, 1, 3])
def test_second_pass_sees_the_update(depth):
    numels, groups = model()
    nd = 4
    M = Mirror(numels, nd, with_acc=False)
    order = fwd_bwd(len(groups))
    s = zsp.Schedule(M.plan, groups, order, depth)
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=dev())
    cs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    s.bind(arena, gs)
    delay = torch.randn(2048, 2048, device=dev(), dtype=torch.bfloat16)
    grads = M.grads(torch.bfloat16, "sched-update")
    gdev = [g.to(dev()) for g in grads]
    torch.cuda.synchronize()
    want1 = expected(M, groups, order)
    caps1 = run_pass(s, cs, True, delay)
    with torch.cuda.stream(cs):
        # a slow compute tail, then the optimizer step; the next pass's
        # gathers must wait for both
        for _ in range(4):
            torch.mm(delay, delay)
        M.plan.reduce_adam_step(zsp.ALL_RANKS, gdev, step=1, stream=cs, **HP)
    for j in range(nd):
        M.o_adam(j, M.o_reduce(j, grads), 1)
    want2 = expected(M, groups, order)
    caps2 = run_pass(s, cs, False, delay)
    check(caps1, want1, f"depth {depth} pass 1")
    check(caps2, want2, f"depth {depth} pass 2 (after Adam)")
    s.destroy()


def test_master_source_and_single_position():
    numels, groups = model()
    M = Mirror(numels, 8, torch.float32, with_acc=False)
    order = [2]
    s = zsp.Schedule(M.plan, groups, order, 3, source="master")
    assert s.info["depth"] == 0
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=dev())
    s.bind(arena, None)
    cs = torch.cuda.current_stream()
    caps = run_pass(s, cs, False, None)
    check(caps, expected(M, groups, order, "master"), "master source")
    s.destroy()


def test_master_source_prefetched():
    numels, groups = model()
    M = Mirror(numels, 8, torch.float32, with_acc=False)
    order = [1, 4, 0, 0, 4, 1]
    s = zsp.Schedule(M.plan, groups, order, 2, source="master")
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=dev())
    cs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    s.bind(arena, gs)
    delay = torch.randn(2048, 2048, device=dev(), dtype=torch.bfloat16)
    caps = run_pass(s, cs, True, delay)
    check(caps, expected(M, groups, order, "master"), "master source, prefetched")
    s.destroy()


def test_order_rules_and_bind_errors():
    numels, groups = model()
    M = Mirror(numels, 4, with_acc=False)
    order = fwd_bwd(len(groups))
    s = zsp.Schedule(M.plan, groups, order, 1)
    arena = torch.empty(s.arena_bytes + 256, dtype=torch.uint8, device=dev())
    gs = torch.cuda.Stream()

    def st(fn, *a):
        try:
            fn(*a)
        except zsp.ZspError as e:
            return e.status
        return 0

    assert st(s.bind, arena[:s.arena_bytes - 1], gs) == binding.ERANGE
    assert st(s.bind, arena[1:1 + s.arena_bytes], gs) == binding.EINVAL   # not 256-aligned
    assert st(s.bind, arena, None) == binding.EINVAL                         # depth 1, no stream
    s.bind(arena, gs)
    assert st(s.acquire, 1) == binding.ESTATE       # out of order
    s.acquire(0)
    assert st(s.acquire, 1) == binding.ESTATE       # 0 still held
    assert st(s.release, 1) == binding.ESTATE       # 1 not held
    s.release(0)
    assert st(s.release, 0) == binding.ESTATE       # already released
    s.acquire(1)
    s.reset()
    assert st(s.acquire, 2) == binding.ESTATE       # reset restarts at 0
    views = s.acquire(0)
    s.release(0)
    torch.cuda.synchronize()
    f, c = groups[order[0]]
    for i, t in enumerate(range(f, f + c)):
        assert_bits(np_of(views[i]), oracle.gather(numels, 4, t, M.o_work), f"after reset {t}")
    s.destroy()
    # a rank-local plan holds one shard only: no gathers
    L = Mirror(numels, 4, rank_local=1, with_acc=False)
    s2 = zsp.Schedule(L.plan, groups, order, 1)
    assert st(s2.bind, torch.empty(s2.arena_bytes, dtype=torch.uint8, device=dev()),
              gs) == binding.ESTATE
    s2.destroy()


@pytest.mark.parametrize("depth", [0, 1, 2])
@pytest.mark.parametrize("slow", [True, False])
@pytest.mark.parametrize("src", ["work", "master"])
def test_copy_engine_every_position(depth, slow, src):
    """The schedule with its gathers on the DMA copy engines (one copy per
    rank's slice of each parameter on the gather stream): each position sees
    its layer bit for bit, over two passes, then after an Adam step."""
    numels, groups = model()
    nd = 8
    M = Mirror(numels, nd, with_acc=False)
    order = fwd_bwd(len(groups))
    s = zsp.Schedule(M.plan, groups, order, depth, source=src)
    s.set_engine("copy")
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=dev())
    cs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    s.bind(arena, gs if depth > 0 else None)
    delay = torch.randn(2048, 2048, device=dev(), dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = expected(M, groups, order, src)
    for rep in range(2):
        caps = run_pass(s, cs, slow, delay)
        check(caps, want, f"copy engine depth {depth} slow {slow} {src} pass {rep}")
    grads = M.grads(torch.bfloat16, ("sched-copy", depth))
    gdev = [g.to(dev()) for g in grads]
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        M.plan.reduce_adam_step(zsp.ALL_RANKS, gdev, step=1, stream=cs, **HP)
    for j in M.ranks:
        M.o_adam(j, M.o_reduce(j, grads), 1)
    caps = run_pass(s, cs, slow, delay)
    check(caps, expected(M, groups, order, src), f"copy engine depth {depth} after update")
    s.destroy()


def test_copy_engine_switch_needs_bind():
    numels, groups = model()
    M = Mirror(numels, 4, with_acc=False)
    s = zsp.Schedule(M.plan, groups, fwd_bwd(len(groups)), 1)
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=dev())
    gs = torch.cuda.Stream()
    s.bind(arena, gs)
    s.acquire(0)
    with pytest.raises(zsp.ZspError) as e:
        s.set_engine("copy")            # a position is held
    assert e.value.status == binding.ESTATE
    s.release(0)
    s.set_engine("copy")
    with pytest.raises(zsp.ZspError) as e:
        s.acquire(0)                    # unbound by the switch
    assert e.value.status == binding.ESTATE
    s.bind(arena, gs)
    views = s.acquire(0)
    s.release(0)
    torch.cuda.synchronize()
    f, c = groups[0]
    for i, t in enumerate(range(f, f + c)):
        assert_bits(np_of(views[i]), oracle.gather(M.numels, M.nd, t, M.o_work), f"param {t}")
    s.destroy()
