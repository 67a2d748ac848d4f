"""Per-layer gather schedule, host side (no GPU): argument checks, the arena
size it asks for, and the order rules that acquire/release enforce before any
device work ("ZeRO Stage 3: Parameter Partitioning", prefetch paragraph;
"ZeRO Stages: Sharding Optimizer State, Gradients, and Parameters", "Stage 3
partitions parameters")."""
import pytest

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import binding

NUMELS = [1000, 7, 3 * 4096, 5, 64, 0, 33]


def status_of(fn, *a, **k):
    try:
        fn(*a, **k)
    except zsp.ZspError as e:
        return e.status
    return 0


def expected_arena(numels, groups, n_steps, depth, esize):
    largest = max(sum(numels[f:f + c]) for f, c in groups)
    slot = (max(largest * esize, 1) + 255) // 256 * 256
    return slot * (min(depth, n_steps - 1) + 1), slot


@pytest.mark.parametrize("depth", [0, 1, 2, 5, 64])
@pytest.mark.parametrize("source,esize", [("work", 2), ("master", 4)])
def test_arena_size(depth, source, esize):
    p = zsp.partition(NUMELS, 4)
    groups = [(0, 2), (2, 3), (5, 2)]
    order = [0, 1, 2, 2, 1, 0]
    s = zsp.Schedule(p, groups, order, depth, source)
    want, slot = expected_arena(NUMELS, groups, len(order), depth, esize)
    assert s.arena_bytes == want
    assert s.info == {"depth": min(depth, len(order) - 1), "slots": min(depth, 5) + 1,
                      "slot_bytes": slot}
    # the slot holds the largest group's unpadded gather, which the oracle's
    # layout gives as a flat range
    L = oracle.Layout(NUMELS, 4)
    for f, c in groups:
        n = sum(L.numel[f:f + c])
        assert n * esize <= slot
    s.destroy()
    p.destroy()


def test_empty_group_still_gets_a_slot():
    p = zsp.partition([0, 0], 2)
    s = zsp.Schedule(p, [(0, 2)], [0], 0)
    assert s.arena_bytes == 256
    s.destroy()


def test_create_errors():
    p = zsp.partition(NUMELS, 4)
    h = p._h
    assert status_of(zsp.zsp_sched_create, h, [(0, 8)], [0], 1) == binding.ERANGE
    assert status_of(zsp.zsp_sched_create, h, [(-1, 1)], [0], 1) == binding.ERANGE
    assert status_of(zsp.zsp_sched_create, h, [(0, 0)], [0], 1) == binding.ERANGE
    assert status_of(zsp.zsp_sched_create, h, [(0, 1)], [1], 1) == binding.ERANGE
    assert status_of(zsp.zsp_sched_create, h, [(0, 1)], [-1], 1) == binding.ERANGE
    assert status_of(zsp.zsp_sched_create, h, [(0, 1)], [0], -1) == binding.EINVAL
    assert status_of(zsp.zsp_sched_create, h, [(0, 1)], [0], 65) == binding.EINVAL
    assert status_of(zsp.zsp_sched_create, h, [], [0], 1) == binding.EINVAL
    assert status_of(zsp.zsp_sched_create, h, [(0, 1)], [], 1) == binding.EINVAL
    assert status_of(zsp.zsp_sched_create, None, [(0, 1)], [0], 1) == binding.EINVAL
    assert "outside" in zsp.last_error() or "NULL" in zsp.last_error()
    p.destroy()


def test_calls_before_bind_fail_without_device_work():
    p = zsp.partition(NUMELS, 4)
    s, _ = zsp.zsp_sched_create(p._h, [(0, 3)], [0, 0], 1)
    # plan has no bound state, so binding the schedule is refused first
    assert binding.lib.zsp_sched_bind(s, None, 0, None) == binding.ESTATE
    assert "every rank" in zsp.last_error()
    out = binding.ctypes.c_void_p()
    assert binding.lib.zsp_sched_acquire(s, 0, None, binding.ctypes.byref(out)) == binding.ESTATE
    assert "zsp_sched_bind" in zsp.last_error()
    assert binding.lib.zsp_sched_release(s, 0, None) == binding.ESTATE
    assert binding.lib.zsp_sched_acquire(s, 0, None, None) == binding.EINVAL
    assert binding.lib.zsp_sched_acquire(None, 0, None, binding.ctypes.byref(out)) == binding.EINVAL
    assert binding.lib.zsp_sched_reset(s) == 0
    assert binding.lib.zsp_sched_reset(None) == binding.EINVAL
    zsp.zsp_sched_destroy(s)
    zsp.zsp_sched_destroy(None)
    p.destroy()


def test_destroying_the_plan_destroys_its_schedules():
    p = zsp.partition(NUMELS, 4)
    s = zsp.Schedule(p, [(0, 3)], [0, 0], 1)
    p.destroy()
    for call in (lambda: s.acquire(0), lambda: s.release(0), s.reset):
        try:
            call()
        except zsp.ZspError as e:
            assert e.status == binding.ESTATE
        else:
            raise AssertionError("a schedule of a destroyed plan must refuse calls")
    s.destroy()   # again: a no-op
    try:
        zsp.Schedule(p, [(0, 3)], [0], 0)
    except zsp.ZspError as e:
        assert e.status == binding.ESTATE
    else:
        raise AssertionError("no schedule on a destroyed plan")
