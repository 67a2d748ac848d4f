"""The hot-path calls under HIP graph capture: no allocation, no host
synchronisation and no memset node inside zsp_reduce_adam_step,
zsp_reduce_shard, zsp_adam_step or zsp_gather_range, so a caller can capture
one step and replay it. Captured once, replayed three times with eager work
and host synchronisations between the replays; after every replay the state
and the gathered parameters equal those of the same calls made eagerly on a
twin plan. The Adam step's scalars are kernel arguments, so a replay repeats
the step number it was captured with (the eager twin does the same). A
prepared list's run (zsp_gather_list_run) is captured the same way. The
layouts take the gather's tile form (long pieces, and a small launch) and
its span form (300 parameters of 64-2000 elements)."""
import pytest
import torch

import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import synth

from test_gpu_parity import HP, Mirror, assert_bits, dev, np_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("numels,nd", [([1003, 64, 5, 0, 3 * 4096 + 1], 4),
                                       ([4096 * 3, 11008 * 2, 4096, 4096], 8),
                                       # short pieces: the range gather's span form
                                       (synth.small_tensor_sizes(count=300, lo=64, hi=2000,
                                                                 seed=21), 8)])
def test_capture_and_replay_matches_eager(numels, nd):
    A, B = Mirror(numels, nd), Mirror(numels, nd)
    grads = [g.to(dev()) for g in A.grads(torch.bfloat16, "graph", poison=False)]
    n_out = max(A.L.total_numel, 8)
    out_a = torch.empty(n_out, dtype=torch.bfloat16, device=dev())
    out_b = torch.empty(n_out, dtype=torch.bfloat16, device=dev())
    T = len(numels)
    torch.cuda.synchronize()

    def step(M, out, stream):
        M.plan.reduce_shard(zsp.ALL_RANKS, grads, accumulate=False, stream=stream)
        M.plan.adam_step(zsp.ALL_RANKS, step=3, stream=stream, **HP)
        M.plan.reduce_adam_step(zsp.ALL_RANKS, grads, step=4, use_acc=True, stream=stream, **HP)
        M.plan.gather_range(0, T, out[:A.L.total_numel], "work", stream=stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(A, out_a, s)
    torch.cuda.synchronize()
    # capture does not run the work: A is still at its copy-in state
    assert_bits(np_of(A.g_master[:A.n]), np_of(B.g_master[:B.n]), "capture ran nothing")
    scratch = torch.empty(1 << 20, device=dev())
    for rep in range(3):
        g.replay()
        step(B, out_b, torch.cuda.current_stream())
        scratch.uniform_()                       # eager work between replays
        torch.cuda.synchronize()
        for name, a, b in (("master", A.g_master, B.g_master), ("m", A.g_m, B.g_m),
                           ("v", A.g_v, B.g_v), ("work", A.g_work, B.g_work),
                           ("acc", A.g_acc, B.g_acc)):
            assert_bits(np_of(a[:A.n]), np_of(b[:B.n]), f"replay {rep}: {name}")
        assert_bits(np_of(out_a[:A.L.total_numel]), np_of(out_b[:B.L.total_numel]),
                    f"replay {rep}: gathered parameters")
    del g


@pytest.mark.parametrize("n_ids", [9, 150])
def test_prepared_list_run_under_capture(n_ids):
    """zsp_gather_list_run captured into a graph (argument form for 9 ids,
    records for 150): each of three replays, after an eager fused step
    between them, gathers the current working copy, bit for bit as an eager
    zsp_gather_many of the same list."""
    from test_gpu_gather_list import outputs
    from zero_sharded_mixed_pad_amd import synth
    numels, nd = synth.small_tensor_sizes(count=160, lo=5, hi=7000, seed=21), 8
    M = Mirror(numels, nd)
    ids = [(7 * i) % M.L.T for i in range(n_ids)]
    got = outputs(M, ids, torch.bfloat16)
    want = outputs(M, ids, torch.bfloat16)
    gl = M.plan.gather_list(ids, got, "work")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            M.plan.gather_prepared(gl, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        grads = [x.to(dev()) for x in M.grads(torch.bfloat16, ("graph-list", rep), poison=False)]
        M.plan.reduce_adam_step(zsp.ALL_RANKS, grads, step=rep + 1, **HP)
        torch.cuda.synchronize()
        g.replay()
        M.plan.gather_many(ids, want, "work")
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, want)):
            n = int(M.L.numel[ids[i]])
            assert_bits(np_of(a[:n]), np_of(b[:n]), f"replay {rep}: entry {i}")
    del g
    gl.close()
