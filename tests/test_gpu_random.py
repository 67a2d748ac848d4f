"""Seeded random cases beyond the hand-picked ones: random parameter lists
(empty, tiny, smaller than N_d, ragged, a few tiles long), random rank counts
up to 64, both gradient dtypes and layouts, with or without an accumulated
micro-batch, on all ranks or one; every step and a gather of a random run of
parameters must match the oracle bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp

from test_gpu_parity import HP, Mirror, assert_bits, dev, np_of

pytestmark = pytest.mark.gpu

ND_CHOICES = [1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 31, 40, 64]


def random_numels(rng):
    kinds = rng.integers(0, 4, size=int(rng.integers(1, 13)))
    out = []
    for k in kinds:
        if k == 0:
            out.append(int(rng.integers(0, 8)))           # empty or below N_d
        elif k == 1:
            out.append(int(rng.integers(8, 700)))         # within a tile
        elif k == 2:
            out.append(int(rng.integers(700, 6000)))      # a few tiles
        else:
            out.append(int(rng.integers(6000, 40000)))    # many tiles
    return out


@pytest.mark.parametrize("seed", range(24))
def test_random_case(seed):
    rng = np.random.default_rng(20261202 + seed)
    numels = random_numels(rng)
    nd = int(rng.choice(ND_CHOICES))
    gdtype = torch.float32 if rng.integers(0, 4) == 0 else torch.bfloat16
    pdtype = torch.float32 if gdtype == torch.float32 else torch.bfloat16
    layout = "shard" if rng.integers(0, 3) == 0 else "full"
    use_acc = bool(rng.integers(0, 2))
    rank = -1 if rng.integers(0, 3) else int(rng.integers(0, nd))
    what = (f"seed {seed}: numels {numels}, N_d {nd}, grads {gdtype}, {layout} layout, "
            f"use_acc {use_acc}, rank {rank}")
    print(f"\n[random] {what}", flush=True)
    M = Mirror(numels, nd, pdtype, seed=seed)
    d = dev()
    ranks = M.ranks if rank < 0 else [rank]
    for step in (1, 2):
        if use_acc:
            g0 = M.grads(gdtype, ("rand-acc", seed, step), layout=layout)
            M.plan.reduce_shard(rank, [g.to(d) for g in g0], layout=layout)
            for j in ranks:
                M.o_acc[M.o_slice(j)] = M.o_reduce(j, g0, layout)
        grads = M.grads(gdtype, ("rand", seed, step), layout=layout)
        M.plan.reduce_adam_step(rank, [g.to(d) for g in grads], step=step, layout=layout,
                                use_acc=use_acc, **HP)
        for j in ranks:
            g = M.o_reduce(j, grads, layout)
            if use_acc:
                acc = M.o_acc[M.o_slice(j)].copy()
                oracle.accumulate(acc, g)
                g = acc
            M.o_adam(j, g, step)
        assert M.check_state(f"{what}, step {step}") == 0, what
    # a random run of consecutive parameters, gathered in one launch
    T = len(numels)
    first = int(rng.integers(0, T))
    n = int(rng.integers(1, T - first + 1))
    total = sum(numels[first:first + n])
    out = torch.empty(max(total, 1), dtype=torch.bfloat16, device=d)
    M.plan.gather_range(first, n, out[:total], "work")
    torch.cuda.synchronize()
    want = [oracle.gather(numels, nd, t, M.o_work) for t in range(first, first + n)]
    want = np.concatenate(want) if want else np.zeros(0, np.uint16)
    assert_bits(np_of(out[:total]), want, f"{what}: gather of [{first}, {first + n})")


def random_groups(rng, T):
    """T parameters cut into consecutive non-empty groups at random points."""
    cuts = sorted(set(int(c) for c in rng.integers(1, T, size=int(rng.integers(0, T)))))
    edges = [0] + cuts + [T]
    return [(a, b - a) for a, b in zip(edges[:-1], edges[1:])]


@pytest.mark.parametrize("seed", range(12))
def test_random_groups_update_and_schedule(seed):
    """Per-group fused updates in a random order cover the model and equal the
    oracle's whole update; then a schedule over the same groups, with a random
    order of positions and depth, hands every position its layer."""
    rng = np.random.default_rng(7_000 + seed)
    numels = random_numels(rng)
    T = len(numels)
    nd = int(rng.choice(ND_CHOICES))
    layout = "shard" if rng.integers(0, 3) == 0 else "full"
    groups = random_groups(rng, T)
    what = f"seed {seed}: numels {numels}, N_d {nd}, {layout} layout, groups {groups}"
    print(f"\n[random groups] {what}", flush=True)
    M = Mirror(numels, nd, seed=100 + seed)
    d = dev()
    for step in (1, 2):
        grads = M.grads(torch.bfloat16, ("rand-groups", seed, step), layout=layout)
        gdev = [g.to(d) for g in grads]
        for gi in rng.permutation(len(groups)):
            first, n = groups[int(gi)]
            M.plan.reduce_adam_step_params(-1, first, n, gdev, step=step, layout=layout, **HP)
        for j in M.ranks:
            M.o_adam(j, M.o_reduce(j, grads, layout), step)
        assert M.check_state(f"{what}, step {step}") == 0, what

    order = [int(g) for g in rng.integers(0, len(groups), size=int(rng.integers(1, 12)))]
    depth = int(rng.integers(0, 4))
    s = zsp.Schedule(M.plan, groups, order, depth)
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=d)
    cs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    s.bind(arena, gs if s.info["depth"] > 0 else None)
    torch.cuda.synchronize()
    caps = []
    with torch.cuda.stream(cs):
        for p in range(len(order)):
            views = s.acquire(p, cs)
            caps.append([v.clone() for v in views])
            s.release(p, cs)
    torch.cuda.synchronize()
    for p, g in enumerate(order):
        first, n = groups[g]
        for i, t in enumerate(range(first, first + n)):
            assert_bits(np_of(caps[p][i]), oracle.gather(numels, nd, t, M.o_work),
                        f"{what}: schedule depth {depth}, position {p}, parameter {t}")
    s.destroy()


@pytest.mark.parametrize("seed", range(12))
def test_random_list_gathers(seed):
    """Random layouts, rank counts and id lists (repeats, empty parameters,
    any order, 1 to 150 entries) gathered one-shot (zsp_gather_many), without
    allocation (zsp_gather_many_noalloc) and prepared (zsp_gather_list_*), from
    the work copy or the master, after a fused step: each output equals the
    oracle's gather of its parameter, bit for bit."""
    rng = np.random.default_rng(20261203 + seed)
    numels = random_numels(rng) + random_numels(rng)
    nd = int(rng.choice([n for n in ND_CHOICES if n <= 40]))
    source = "master" if rng.integers(0, 3) == 0 else "work"
    n_ids = int(rng.choice([1, 5, 64, 65, 150]))
    ids = [int(x) for x in rng.integers(0, len(numels), size=n_ids)]
    print(f"\n[random list] seed {seed}: {len(numels)} parameters, N_d {nd}, {source}, "
          f"{n_ids} ids", flush=True)
    M = Mirror(numels, nd, seed=seed)
    d = dev()
    grads = M.grads(torch.bfloat16, ("rand-list", seed))
    M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(d) for g in grads], step=1, **HP)
    for j in M.ranks:
        M.o_adam(j, M.o_reduce(j, grads), 1)
    dt = torch.bfloat16 if source == "work" else torch.float32
    src = M.o_work if source == "work" else M.o_master
    gl_outs = [torch.full((max(int(M.L.numel[t]), 1),), float("nan"), dtype=dt, device=d)
               for t in ids]
    gl = M.plan.gather_list(ids, gl_outs, source)
    for form in ("many", "noalloc", "prepared"):
        outs = gl_outs if form == "prepared" else [
            torch.full((max(int(M.L.numel[t]), 1),), float("nan"), dtype=dt, device=d)
            for t in ids]
        if form == "many":
            M.plan.gather_many(ids, outs, source)
        elif form == "noalloc":
            M.plan.gather_many_noalloc(ids, outs, source)
        else:
            M.plan.gather_prepared(gl)
        torch.cuda.synchronize()
        for i, (t, o) in enumerate(zip(ids, outs)):
            n = int(M.L.numel[t])
            if n:
                assert_bits(np_of(o[:n]), oracle.gather(M.numels, M.nd, t, src),
                            f"seed {seed}, {form}: entry {i} (id {t})")
    gl.close()
