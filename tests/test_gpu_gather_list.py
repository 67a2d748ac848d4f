"""zsp_gather_many: a list of parameter ids, in any order and with repeats,
each gathered into its own separately allocated output, bit for bit against
the oracle's gather of the same parameter ("The ZeRO-3 Diagram Most People
Remember Is Wrong", section 3: a module's parameters are gathered just
before it runs; section 8: gathers go out in buckets of parameters).

Lists of up to 64 non-empty parameters run from the kernel arguments;
longer ones are staged through the plan's slots (both forms are covered,
including more staged calls than there are slots, on two streams). Every
output is allocated with a guard zone behind it that must keep its fill.
"""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import synth

from test_gpu_parity import Mirror, assert_bits, np_of

pytestmark = pytest.mark.gpu

GUARD = 40


def dev():
    return torch.device("cuda")


def outputs(M, ids, dtype):
    """One fresh tensor per id: numel elements plus a guard zone, all NaN."""
    return [torch.full((int(M.L.numel[t]) + GUARD,), float("nan"), dtype=dtype, device=dev())
            for t in ids]


def check(M, ids, outs, source, what):
    torch.cuda.synchronize()
    src = M.o_work if source == "work" else M.o_master
    for i, (t, o) in enumerate(zip(ids, outs)):
        n = int(M.L.numel[t])
        got = np_of(o)
        assert_bits(got[:n], oracle.gather(M.numels, M.nd, t, src), f"{what}: entry {i} (id {t})")
        tail = got[n:]
        tail_f = oracle.bf16_to_f32(tail) if tail.dtype == np.uint16 else tail
        assert np.isnan(tail_f).all(), f"{what}: entry {i} wrote past its {n} elements"


LAYOUTS = {
    "short": (synth.small_tensor_sizes(count=200, lo=5, hi=2000, seed=9), 8),
    "long": ([512 * 300, 4096 * 37 + 5, 100003, 77, 262144 + 13, 512 * 64, 9000], 8),
    "mixed": ([1003, 64, 5, 0, 3 * 4096 + 1, 0, 7, 70000], 4),
    "many_ranks": ([3] * 40 + [1000, 5000, 0, 12345], 64),
    "wide": ([300, 7, 5000, 1 << 16], 256),
    "ragged": ([511 * 8, 512 * 8, 513 * 8, 8 * 8 * 64 + 3, 1, 2], 8),
    "small_tensors": (synth.small_tensor_sizes(count=300, lo=8, hi=3000, seed=5), 8),
}


def id_lists(T, rng):
    lists = {
        "ascending": list(range(T)),
        "reversed": list(range(T - 1, -1, -1)),
        "random_repeats": [int(x) for x in rng.integers(0, T, size=2 * T + 3)],
        "every_third": list(range(1, T, 3)),
        "single": [T - 1],
        "empty": [],
    }
    perm = [int(x) for x in rng.permutation(T)]
    lists["permuted_prefix"] = perm[: max(1, T // 2)]
    return lists


@pytest.mark.parametrize("which", list(LAYOUTS))
@pytest.mark.parametrize("source", ["work", "master"])
def test_lists_match_oracle(which, source):
    numels, nd = LAYOUTS[which]
    print(f"\n[gather list] layout {which}, source {source}", flush=True)
    M = Mirror(numels, nd)
    rng = np.random.default_rng(synth.derive_seed("gather-list", which))
    dt = torch.bfloat16 if source == "work" else torch.float32
    for name, ids in id_lists(M.L.T, rng).items():
        outs = outputs(M, ids, dt)
        M.plan.gather_many(ids, outs, source)
        check(M, ids, outs, source, f"{which}/{name}")


def test_staged_lists_on_two_streams():
    """Twelve staged lists (more than the four slots) alternating between two
    streams, each output checked: a slot is never refilled under a gather
    that still reads it."""
    numels, nd = synth.small_tensor_sizes(count=400, lo=5, hi=5000, seed=11), 8
    M = Mirror(numels, nd)
    rng = np.random.default_rng(3)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    jobs = []
    for k in range(12):
        ids = [int(x) for x in rng.integers(0, M.L.T, size=int(rng.integers(65, 400)))]
        outs = outputs(M, ids, torch.bfloat16)
        torch.cuda.synchronize()
        M.plan.gather_many(ids, outs, "work", stream=streams[k % 2])
        jobs.append((ids, outs))
    for k, (ids, outs) in enumerate(jobs):
        check(M, ids, outs, "work", f"staged call {k}")


def test_list_equals_range_form_after_steps():
    """After fused steps, the list form over every parameter into separate
    outputs equals the range form into one buffer, for the work copy, the
    master and the accumulator."""
    numels, nd = [1003, 64, 5, 0, 3 * 4096 + 1, 12345, 77], 4
    M = Mirror(numels, nd)
    d = dev()
    for step in (1, 2):
        grads = M.grads(torch.bfloat16, ("list", step))
        M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(d) for g in grads], step=step,
                                lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
        M.plan.reduce_shard(zsp.ALL_RANKS, [g.to(d) for g in grads])
    L = M.L
    for source, dt in (("work", torch.bfloat16), ("master", torch.float32),
                       ("acc", torch.float32)):
        whole = torch.empty(L.total_numel, dtype=dt, device=d)
        M.plan.gather_range(0, L.T, whole, source)
        ids = list(range(L.T - 1, -1, -1))
        outs = outputs(M, ids, dt)
        M.plan.gather_many(ids, outs, source)
        torch.cuda.synchronize()
        for t, o in zip(ids, outs):
            a, b = int(L.flat_off[t]), int(L.flat_off[t + 1])
            assert torch.equal(o[:b - a].view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                               whole[a:b].view(torch.int16 if dt == torch.bfloat16 else torch.int32)), \
                f"{source}: parameter {t}"


def test_staged_list_in_several_chunks():
    """A staged list whose tiles exceed one slot's record area (2^19 tiles)
    runs in several pairs of launches; gather(partition(x)) == x for every
    output."""
    numels = [300_000_000] + [4096 + 3 * i for i in range(70)]
    nd = 8
    plan = zsp.partition(numels, nd)
    d = dev()
    n = nd * plan.S
    master = torch.empty(n, dtype=torch.float32, device=d)
    m = torch.empty_like(master)
    v = torch.empty_like(master)
    work = torch.empty(n, dtype=torch.bfloat16, device=d)
    plan.bind_state(zsp.ALL_RANKS, master, m, v, work)
    flat = synth.normal(plan.total_numel, 0.02, torch.bfloat16, synth.derive_seed("chunks", 0), d)
    plan.load_params(flat)
    ids = list(range(len(numels) - 1, -1, -1))   # 71 entries: staged
    outs = [torch.empty(numels[t], dtype=torch.bfloat16, device=d) for t in ids]
    plan.gather_many(ids, outs, "work")
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(numels)])
    for t, o in zip(ids, outs):
        want = flat[int(offs[t]):int(offs[t + 1])]
        assert torch.equal(o.view(torch.int16), want.view(torch.int16)), f"parameter {t}"
    plan.destroy()


def test_list_argument_errors():
    numels, nd = [1003, 64, 0], 4
    M = Mirror(numels, nd)
    d = dev()
    ok = torch.empty(2048, dtype=torch.bfloat16, device=d)
    with pytest.raises(zsp.ZspError) as e:
        M.plan.gather_many([0, 3], [ok, ok])
    assert e.value.status == zsp.binding.ERANGE
    with pytest.raises(zsp.ZspError) as e:
        M.plan.gather_many([-1], [ok])
    assert e.value.status == zsp.binding.ERANGE
    with pytest.raises(zsp.ZspError) as e:
        M.plan.gather_many([1], [ok[1:]])   # misaligned output
    assert e.value.status == zsp.binding.EINVAL
    with pytest.raises(zsp.ZspError) as e:
        M.plan.gather_many([1, 0], [ok, None])
    assert e.value.status == zsp.binding.EINVAL
    no_acc = Mirror(numels, nd, with_acc=False)
    with pytest.raises(zsp.ZspError) as e:
        no_acc.plan.gather_many([0], [torch.empty(2048, dtype=torch.float32, device=d)], "acc")
    assert e.value.status == zsp.binding.ESTATE
    # an empty parameter needs no output; an empty list does nothing
    M.plan.gather_many([2], [None])
    M.plan.gather_many([], [])
    local = Mirror(numels, nd, rank_local=1)
    with pytest.raises(zsp.ZspError) as e:
        local.plan.gather_many([0], [ok])
    assert e.value.status == zsp.binding.ESTATE
    M.check_state("after rejected list gathers", exact=True)


def test_prepared_list_after_each_step():
    """A list marshalled once (GatherList) and run after each of three fused
    steps returns the current working copy each time, for an argument-form
    and a staged list."""
    numels, nd = synth.small_tensor_sizes(count=120, lo=5, hi=9000, seed=4), 8
    M = Mirror(numels, nd)
    d = dev()
    short_ids = list(range(0, M.L.T, 3))[:40]          # argument form
    long_ids = list(range(M.L.T - 1, -1, -1))          # staged
    lists = []
    for ids in (short_ids, long_ids):
        outs = outputs(M, ids, torch.bfloat16)
        lists.append((ids, outs, M.plan.gather_list(ids, outs, "work")))
    for step in (1, 2, 3):
        grads = M.grads(torch.bfloat16, ("prepared", step))
        M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(d) for g in grads], step=step,
                                lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
        for j in M.ranks:
            M.o_adam(j, M.o_reduce(j, grads), step)
        for ids, outs, gl in lists:
            M.plan.gather_prepared(gl)
            check(M, ids, outs, "work", f"prepared list of {len(ids)}, step {step}")


@pytest.mark.parametrize("which", list(LAYOUTS))
@pytest.mark.parametrize("source", ["work", "master", "acc"])
def test_prepared_lists_match_oracle(which, source):
    """zsp_gather_list_create / _run: each id list of test_lists_match_oracle,
    prepared once and run twice (the second run into outputs refilled with
    NaN), equals the oracle's gather; the accumulator source against the
    range form."""
    numels, nd = LAYOUTS[which]
    print(f"\n[prepared list] layout {which}, source {source}", flush=True)
    M = Mirror(numels, nd)
    d = dev()
    if source == "acc":
        grads = M.grads(torch.bfloat16, ("prepared-acc", which))
        M.plan.reduce_shard(zsp.ALL_RANKS, [g.to(d) for g in grads])
        whole = torch.empty(max(M.L.total_numel, 1), dtype=torch.float32, device=d)
        M.plan.gather_range(0, M.L.T, whole, "acc")
    rng = np.random.default_rng(synth.derive_seed("prepared-list", which))
    dt = torch.bfloat16 if source == "work" else torch.float32
    for name, ids in id_lists(M.L.T, rng).items():
        outs = outputs(M, ids, dt)
        gl = M.plan.gather_list(ids, outs, source)
        for run in (0, 1):
            if run:
                for o in outs:
                    o.fill_(float("nan"))
            M.plan.gather_prepared(gl)
            if source == "acc":
                torch.cuda.synchronize()
                for i, (t, o) in enumerate(zip(ids, outs)):
                    a, b = int(M.L.flat_off[t]), int(M.L.flat_off[t + 1])
                    assert torch.equal(o[:b - a].view(torch.int32), whole[a:b].view(torch.int32)), \
                        f"{which}/{name} run {run}: entry {i} (id {t})"
                    assert torch.isnan(o[b - a:]).all(), f"{which}/{name}: entry {i} overran"
            else:
                check(M, ids, outs, source, f"{which}/{name} run {run}")
        gl.close()
        gl.close()   # a second close is a no-op


def test_prepared_list_streams_and_rebinding():
    """A prepared staged list runs on two other streams, and after the state
    is bound again to new tensors (same layout) it reads the new binding."""
    numels, nd = synth.small_tensor_sizes(count=150, lo=5, hi=6000, seed=12), 8
    M = Mirror(numels, nd)
    d = dev()
    ids = [int(x) for x in np.random.default_rng(8).permutation(M.L.T)]
    outs = outputs(M, ids, torch.bfloat16)
    gl = M.plan.gather_list(ids, outs, "work")
    for s in (torch.cuda.Stream(), torch.cuda.Stream()):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        M.plan.gather_prepared(gl, stream=s)
        check(M, ids, outs, "work", "prepared list on a side stream")
    # bind fresh state tensors, load other parameters, run the same list
    n = nd * M.plan.S
    st = [torch.empty(n, dtype=torch.float32, device=d) for _ in range(3)]
    work = torch.empty(n, dtype=torch.bfloat16, device=d)
    M.plan.bind_state(zsp.ALL_RANKS, st[0], st[1], st[2], work)
    flat = synth.normal(M.plan.total_numel, 0.02, torch.bfloat16, synth.derive_seed("rebind", 0), d)
    M.plan.load_params(flat)
    M.plan.gather_prepared(gl)
    torch.cuda.synchronize()
    for i, (t, o) in enumerate(zip(ids, outs)):
        a, b = int(M.L.flat_off[t]), int(M.L.flat_off[t + 1])
        assert torch.equal(o[:b - a].view(torch.int16), flat[a:b].view(torch.int16)), \
            f"after rebinding: entry {i} (id {t})"
    # bound for one rank only: the list cannot run
    local = torch.empty(M.plan.S, dtype=torch.float32, device=d)
    M.plan.bind_state(0, local, torch.empty_like(local), torch.empty_like(local),
                      torch.empty(M.plan.S, dtype=torch.bfloat16, device=d))
    with pytest.raises(zsp.ZspError) as e:
        M.plan.gather_prepared(gl)
    assert e.value.status == zsp.binding.ESTATE
    gl.close()
    with pytest.raises(ValueError):
        gl.run()


def test_prepared_list_errors():
    """Create takes zsp_gather_many's checks; run needs a list."""
    numels, nd = [1003, 64, 0], 4
    M = Mirror(numels, nd)
    d = dev()
    ok = torch.empty(2048, dtype=torch.bfloat16, device=d)
    for ids, outs, status in (([0, 3], [ok, ok], zsp.binding.ERANGE),
                              ([1], [ok[1:]], zsp.binding.EINVAL),
                              ([1, 0], [ok, None], zsp.binding.EINVAL)):
        with pytest.raises(zsp.ZspError) as e:
            M.plan.gather_list(ids, outs, "work")
        assert e.value.status == status
    no_acc = Mirror(numels, nd, with_acc=False)
    with pytest.raises(zsp.ZspError) as e:
        no_acc.plan.gather_list([0], [torch.empty(2048, dtype=torch.float32, device=d)], "acc")
    assert e.value.status == zsp.binding.ESTATE
    assert zsp.binding.lib.zsp_gather_list_run(None, None) == zsp.binding.EINVAL
    zsp.binding.lib.zsp_gather_list_destroy(None)
    empty = M.plan.gather_list([2], [None], "work")   # nothing to gather
    M.plan.gather_prepared(empty)
    empty.close()
    M.check_state("after rejected prepared lists", exact=True)


def test_prepared_list_beyond_one_slot():
    """A prepared list of more tiles than one staging slot's record area
    (2^19 tiles) keeps the records of all of them; gather(partition(x)) == x
    for every output."""
    numels = [300_000_000] + [4096 + 3 * i for i in range(70)]
    nd = 8
    plan = zsp.partition(numels, nd)
    d = dev()
    n = nd * plan.S
    master = torch.empty(n, dtype=torch.float32, device=d)
    m = torch.empty_like(master)
    v = torch.empty_like(master)
    work = torch.empty(n, dtype=torch.bfloat16, device=d)
    plan.bind_state(zsp.ALL_RANKS, master, m, v, work)
    flat = synth.normal(plan.total_numel, 0.02, torch.bfloat16, synth.derive_seed("chunks", 1), d)
    plan.load_params(flat)
    ids = list(range(len(numels) - 1, -1, -1))
    outs = [torch.empty(numels[t], dtype=torch.bfloat16, device=d) for t in ids]
    gl = plan.gather_list(ids, outs, "work")
    plan.gather_prepared(gl)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(numels)])
    for t, o in zip(ids, outs):
        want = flat[int(offs[t]):int(offs[t + 1])]
        assert torch.equal(o.view(torch.int16), want.view(torch.int16)), f"parameter {t}"
    gl.close()
    plan.destroy()
