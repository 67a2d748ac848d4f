"""zsp_gather_many_noalloc against zsp_gather_many: the same lists into
separate outputs give the same bits, on two calls in a row, the second with
a smaller list (the device array keeps the first call's contents, which the
second must not depend on), through the C ABI. Both are also checked
against the oracle's gather. A short list (kernel-argument form, no
staging), an over-long list (ZSP_ERANGE) and a second plan on the same
array follow."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import binding, synth

from test_gpu_parity import Mirror, assert_bits, np_of

pytestmark = pytest.mark.gpu


def c_call(fn, plan, ids, outs, src=binding.SRC_WORK):
    n = len(ids)
    ids_c = (ctypes.c_int32 * max(n, 1))(*ids)
    outs_c = (ctypes.c_void_p * max(n, 1))(*[o.data_ptr() if o is not None else None
                                             for o in outs])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(plan.handle, ids_c, n, src, outs_c, stream)


def fresh(M, ids, fill=float("nan")):
    return [torch.full((int(M.L.numel[t]) + 16,), fill, dtype=torch.bfloat16, device="cuda")
            for t in ids]


def same_bits(a_outs, b_outs, M, ids, what):
    torch.cuda.synchronize()
    for i, (t, a, b) in enumerate(zip(ids, a_outs, b_outs)):
        n = int(M.L.numel[t])
        assert torch.equal(a[:n].view(torch.int16), b[:n].view(torch.int16)), f"{what}: entry {i}"
        assert_bits(np_of(a[:n]), oracle.gather(M.numels, M.nd, t, M.o_work), f"{what}: oracle {i}")
        assert torch.isnan(a[n:].float()).all(), f"{what}: entry {i} wrote past its end"


def test_noalloc_matches_gather_many_twice_then_smaller():
    numels, nd = synth.small_tensor_sizes(count=600, lo=5, hi=20000, seed=21), 8
    print("\n[no-alloc] 600 tensors, N_d = 8", flush=True)
    M = Mirror(numels, nd)
    rng = np.random.default_rng(5)
    L = M.L
    first = [int(x) for x in rng.permutation(L.T)][:500]          # staged, 500 entries
    second = [int(x) for x in rng.integers(0, L.T, size=90)]      # staged, smaller
    for k, ids in enumerate((first, second)):
        want = fresh(M, ids)
        assert c_call(binding.lib.zsp_gather_many, M.plan, ids, want) == binding.OK
        got = fresh(M, ids)
        st = c_call(binding.lib.zsp_gather_many_noalloc, M.plan, ids, got)
        assert st == binding.OK, zsp.last_error()
        same_bits(got, want, M, ids, f"call {k + 1} ({len(ids)} entries)")


def test_noalloc_short_list_and_limits():
    numels, nd = [1003, 64, 0, 3 * 4096 + 1, 77777], 4
    M = Mirror(numels, nd)
    ids = [4, 2, 0, 3]                                             # argument form
    want = fresh(M, ids)
    assert c_call(binding.lib.zsp_gather_many, M.plan, ids, want) == binding.OK
    got = fresh(M, ids)
    assert c_call(binding.lib.zsp_gather_many_noalloc, M.plan, ids, got) == binding.OK
    same_bits(got, want, M, ids, "short list")
    # more non-empty entries than the array holds: refused, nothing enqueued
    big = [0] * 65537
    outs = (ctypes.c_void_p * len(big))(*([want[2].data_ptr()] * len(big)))
    ids_c = (ctypes.c_int32 * len(big))(*big)
    st = binding.lib.zsp_gather_many_noalloc(M.plan.handle, ids_c, len(big), binding.SRC_WORK,
                                            outs, ctypes.c_void_p(0))
    assert st == binding.ERANGE and "at most" in zsp.last_error()


def test_noalloc_second_plan_same_array():
    """Two plans on one GPU share the array; calls on one stream, one after
    the other, each give their own plan's parameters."""
    A = Mirror(synth.small_tensor_sizes(count=200, lo=5, hi=3000, seed=1), 8, seed=1)
    B = Mirror(synth.small_tensor_sizes(count=150, lo=100, hi=9000, seed=2), 16, seed=2)
    ida = list(range(A.L.T - 1, -1, -1))
    idb = list(range(B.L.T))
    ga, gb = fresh(A, ida), fresh(B, idb)
    assert c_call(binding.lib.zsp_gather_many_noalloc, A.plan, ida, ga) == binding.OK
    assert c_call(binding.lib.zsp_gather_many_noalloc, B.plan, idb, gb) == binding.OK
    wa, wb = fresh(A, ida), fresh(B, idb)
    assert c_call(binding.lib.zsp_gather_many, A.plan, ida, wa) == binding.OK
    assert c_call(binding.lib.zsp_gather_many, B.plan, idb, wb) == binding.OK
    same_bits(ga, wa, A, ida, "plan A")
    same_bits(gb, wb, B, idb, "plan B")
