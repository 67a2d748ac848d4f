"""C ABI checks that need no GPU: the library loads and exports every entry
point include/zsp.h declares, its host-side layout tables equal the oracle's
bit for bit, and argument errors come back as the documented status codes
before anything touches a device."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "zsp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zsp_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "zsp_reduce_adam_step" in names and "zsp_gather" in names
    lib = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in zsp.h but not exported"


def test_binding_covers_every_entry_point():
    for n in declared_functions():
        if n == "zsp_last_error":
            assert callable(zsp.last_error)
        else:
            assert callable(getattr(binding, n)), n


LAYOUT_CASES = [
    ([1000 * 1003], 4), ([1001 * 1003], 4), ([1000 * 1003], 16), ([0, 1, 2, 3, 4, 5], 8),
    ([4096 * 4096] * 4 + [4096 * 11008] * 3 + [4096] * 2, 8), ([7] * 50, 256), ([1], 1),
    (synth.small_tensor_sizes()[:2000], 8),
]


@pytest.mark.parametrize("numels,nd", LAYOUT_CASES)
def test_layout_tables_match_oracle(numels, nd):
    plan = zsp.partition(numels, nd)
    L = oracle.Layout(numels, nd)
    info = plan.info()
    assert info["shard_elems"] == L.S
    assert info["total_padded"] == L.total_padded
    assert plan.total_numel == L.total_numel
    assert info["model_state_bytes_per_rank"] == oracle.model_state_bytes(L.S)
    for t in range(len(numels)):
        d = plan.tensor(t)
        assert d["numel"] == numels[t]
        assert d["pad"] == L.pad[t]
        assert d["shard_len"] == L.shard_len[t]
        assert d["full_off"] == L.full_off[t]
        assert d["shard_off"] == L.shard_off[t]
        assert d["flat_off"] == L.flat_off[t]
    plan.destroy()


def test_small_tensor_workload_is_mostly_padded():
    """The 10,000-tensor workload exercises per-tensor padding heavily."""
    sizes = synth.small_tensor_sizes()
    L = oracle.Layout(sizes, 8)
    assert len(sizes) == 10_000 and min(sizes) >= 64 and max(sizes) <= 65536
    assert (L.pad > 0).mean() > 0.8


def _status(fn, *args):
    try:
        fn(*args)
    except zsp.ZspError as e:
        return e.status
    return 0


def test_partition_argument_errors():
    assert _status(zsp.zsp_partition, [5], 0) == binding.EINVAL
    assert _status(zsp.zsp_partition, [5], 257) == binding.EINVAL
    assert _status(zsp.zsp_partition, [5, -1], 2) == binding.EINVAL
    assert _status(zsp.zsp_partition, [], 2) == binding.EINVAL
    assert _status(zsp.zsp_partition, [1 << 61], 2) == binding.ERANGE
    lib = binding.lib
    h = ctypes.c_void_p()
    assert lib.zsp_partition(None, 1, 2, ctypes.byref(h)) == binding.EINVAL
    arr = (ctypes.c_int64 * 1)(5)
    assert lib.zsp_partition(arr, 1, 2, None) == binding.EINVAL
    assert "out is NULL" in zsp.last_error()


def test_query_errors():
    lib = binding.lib
    plan = zsp.partition([5, 6], 3)
    assert _status(zsp.zsp_plan_tensor, plan.handle, 2) == binding.ERANGE
    assert _status(zsp.zsp_plan_tensor, plan.handle, -1) == binding.ERANGE
    assert lib.zsp_plan_info(None, None, None, None) == binding.EINVAL
    assert lib.zsp_plan_info(plan.handle, None, None, None) == binding.OK
    lib.zsp_destroy(None)  # ignored
    plan.destroy()


def test_unbound_calls_fail_before_touching_a_device():
    lib = binding.lib
    plan = zsp.partition([5, 6], 3)
    h = plan.handle
    grads = (ctypes.c_void_p * 3)(16, 32, 48)
    null = ctypes.c_void_p()
    assert lib.zsp_load_params(h, ctypes.c_void_p(256), binding.F32, null) == binding.ESTATE
    assert lib.zsp_reduce_shard(h, -1, grads, binding.BF16, 0, 0, null) == binding.ESTATE
    assert lib.zsp_adam_step(h, -1, 1e-3, 0.9, 0.999, 1e-8, 1, null) == binding.ESTATE
    assert lib.zsp_reduce_adam_step(h, -1, grads, binding.BF16, 0, 0, 1e-3, 0.9, 0.999, 1e-8,
                                    1, null) == binding.ESTATE
    assert lib.zsp_gather(h, 0, binding.SRC_WORK, ctypes.c_void_p(256), null) == binding.ESTATE
    assert lib.zsp_gather(h, 9, binding.SRC_WORK, ctypes.c_void_p(256), null) == binding.ERANGE
    assert lib.zsp_gather_range(h, 0, 1, binding.SRC_WORK, ctypes.c_void_p(256),
                                null) == binding.ESTATE
    ids = (ctypes.c_int32 * 2)(1, 0)
    outs = (ctypes.c_void_p * 2)(256, 512)
    assert lib.zsp_gather_many(h, ids, 2, binding.SRC_WORK, outs, null) == binding.ESTATE
    assert "bind" in zsp.last_error()
    gl = ctypes.c_void_p(1234)
    assert lib.zsp_gather_list_create(h, ids, 2, binding.SRC_WORK, outs, null,
                                      ctypes.byref(gl)) == binding.ESTATE
    assert gl.value is None                       # *list cleared on failure
    assert lib.zsp_gather_list_create(h, ids, 2, binding.SRC_WORK, outs, null,
                                      None) == binding.EINVAL
    assert lib.zsp_gather_list_run(None, null) == binding.EINVAL
    lib.zsp_gather_list_destroy(None)             # ignored
    assert lib.zsp_reduce_shard(None, -1, grads, 1, 0, 0, null) == binding.EINVAL
    plan.destroy()


def test_bind_argument_errors_before_device_use():
    lib = binding.lib
    plan = zsp.partition([5, 6], 3)
    h = plan.handle
    p = [ctypes.c_void_p(256 * (i + 1)) for i in range(5)]
    assert lib.zsp_bind_state(h, 3, *p) == binding.EINVAL          # rank outside [0, 3)
    assert lib.zsp_bind_state(h, -2, *p) == binding.EINVAL
    bad = list(p)
    bad[2] = ctypes.c_void_p(256 + 4)                               # v misaligned
    assert lib.zsp_bind_state(h, -1, *bad) == binding.EINVAL
    assert "v is not 16-byte aligned" in zsp.last_error()
    bad = list(p)
    bad[0] = ctypes.c_void_p()                                      # master NULL
    assert lib.zsp_bind_state(h, -1, *bad) == binding.EINVAL
    bad = list(p)
    bad[4] = ctypes.c_void_p(256 + 8)                               # grad_acc misaligned
    assert lib.zsp_bind_state(h, -1, *bad) == binding.EINVAL
    plan.destroy()


try:
    from hypothesis import given, settings, strategies as st
except ImportError:  # the property test below needs hypothesis
    given = None


if given is not None:
    @settings(max_examples=300, deadline=None)
    @given(numels=st.lists(st.one_of(st.integers(0, 9), st.integers(0, 5000),
                                     st.integers(0, 10 ** 12)), min_size=1, max_size=40),
           nd=st.integers(1, 256))
    def test_layout_queries_match_oracle_on_random_lists(numels, nd):
        """The library's layout queries equal the oracle's tables for random
        parameter lists (sizes from empty to 10^12 elements, any rank count
        the library accepts)."""
        plan = zsp.partition(numels, nd)
        L = oracle.Layout(numels, nd)
        info = plan.info()
        assert (info["shard_elems"], info["total_padded"], plan.total_numel) == (
            L.S, L.total_padded, L.total_numel)
        for t in range(len(numels)):
            d = plan.tensor(t)
            assert (d["pad"], d["shard_len"], d["full_off"], d["shard_off"], d["flat_off"]) == (
                L.pad[t], L.shard_len[t], L.full_off[t], L.shard_off[t], L.flat_off[t])
        plan.destroy()
