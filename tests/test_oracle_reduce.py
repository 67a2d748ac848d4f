"""Pins for the oracle's shard reduce and micro-batch accumulation.

The reduce is a plain sum over ranks in fp32, in rank order 0..N_d-1. It is
pinned by special cases whose results IEEE arithmetic fixes exactly (N_d=1,
equal inputs, crafted order probes, signed zeros), by the exact sum within
the classical error bound of recursive summation, and by a list-based brute
force of which gradient element lands in which shard slot.
"""
import math

import numpy as np
import pytest
import torch

import oracle

U = 2.0 ** -24  # unit roundoff of fp32


def bf16_bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_single_rank_is_identity():
    numels = [10, 7, 1]
    L = oracle.Layout(numels, 1)
    g = (np.random.default_rng(0).standard_normal(L.total_padded) * 1e-2).astype(np.float32)
    out = oracle.reduce(numels, 1, 0, [g])
    assert np.array_equal(out.view(np.uint32), g.view(np.uint32))
    gb = bf16_bits(g)
    outb = oracle.reduce(numels, 1, 0, [gb])
    assert np.array_equal(outb, oracle.bf16_to_f32(gb))


@pytest.mark.parametrize("nd", [2, 3, 8, 16, 64])
def test_equal_inputs_give_exact_multiple(nd):
    """Adding a bf16 value n times is exact in fp32 for n < 2^16 (8 + 16
    significant bits fit in 24), so the sum is n*g exactly."""
    numels = [257, 64]
    L = oracle.Layout(numels, nd)
    g = bf16_bits(np.random.default_rng(nd).standard_normal(L.total_padded) * 1e-3)
    out = np.stack([oracle.reduce(numels, nd, j, [g] * nd) for j in range(nd)])
    ref = [oracle.gather(numels, nd, t, out.reshape(-1)) for t in range(len(numels))]
    flatg = oracle.bf16_to_f32(g).astype(np.float64)
    for t in range(len(numels)):
        seg = flatg[L.full_off[t]:L.full_off[t] + numels[t]]
        assert np.array_equal(ref[t].astype(np.float64), nd * seg)


def test_rank_order_probe():
    """1 + 2^-24 rounds back to 1 (tie, even), so 1, 2^-24, 2^-24 in rank
    order sums to exactly 1; with the small values first the sum is
    1 + 2^-23. A different summation order or tree would change the bits."""
    one, tiny = np.float32(1.0), np.float32(2.0 ** -24)
    big_first = [np.array([one], np.float32), np.array([tiny], np.float32),
                 np.array([tiny], np.float32)]
    out = oracle.reduce([3], 3, 0, [np.repeat(b, 3) for b in big_first])
    assert out[0] == np.float32(1.0)
    small_first = big_first[::-1]
    out = oracle.reduce([3], 3, 0, [np.repeat(b, 3) for b in small_first])
    assert out[0] == np.float32(1.0 + 2.0 ** -23)


def test_sum_starts_from_rank_zero():
    """-0 + -0 = -0, but +0 + -0 = +0: the sum begins with rank 0's value
    rather than with a +0 accumulator."""
    g = [np.full(2, -0.0, np.float32) for _ in range(2)]
    out = oracle.reduce([2], 2, 0, g)
    assert out.view(np.uint32)[0] == 0x80000000


@pytest.mark.parametrize("nd,dtype", [(2, "f32"), (3, "bf16"), (8, "bf16"),
                                      (16, "bf16"), (8, "f32"), (64, "bf16")])
def test_within_recursive_summation_bound(nd, dtype):
    """|fl(sum) - sum| <= (n-1) u sum|g_r| for left-to-right summation
    (Higham, Accuracy and Stability of Numerical Algorithms, section 4.2),
    with the exact sum from math.fsum."""
    numels = [300, 45]
    L = oracle.Layout(numels, nd)
    rng = np.random.default_rng(nd)
    grads = [(rng.standard_normal(L.total_padded) * 1e-3).astype(np.float32)
             for _ in range(nd)]
    if dtype == "bf16":
        grads = [bf16_bits(g) for g in grads]
    vals = [oracle.bf16_to_f32(g) if dtype == "bf16" else g for g in grads]
    for j in range(nd):
        out = oracle.reduce(numels, nd, j, grads)
        for t in range(len(numels)):
            s = int(L.shard_len[t])
            for i in range(s):
                k = j * s + i
                e = int(L.shard_off[t]) + i
                if k >= numels[t]:
                    assert out[e].view(np.uint32) == 0
                    continue
                src = int(L.full_off[t]) + k
                terms = [float(v[src]) for v in vals]
                exact = math.fsum(terms)
                bound = (nd - 1) * U * math.fsum(abs(x) for x in terms) * (1 + 1e-6)
                assert abs(float(out[e]) - exact) <= bound


def brute_expected(numels, nd, j, grads_by_tensor):
    """Expected shard of rank j from per-tensor padded gradient lists, summed
    one fp32 addition at a time in rank order; pads give +0."""
    out = []
    for t, n in enumerate(numels):
        padded_len = n
        while padded_len % nd:
            padded_len += 1
        s = padded_len // nd
        for k in range(j * s, (j + 1) * s):
            if k >= n:
                out.append(np.float32(0.0))
                continue
            acc = np.float32(grads_by_tensor[0][t][k])
            for r in range(1, nd):
                acc = np.float32(acc + np.float32(grads_by_tensor[r][t][k]))
            out.append(acc)
    return np.array(out, np.float32)


@pytest.mark.parametrize("numels,nd", [([10, 7, 0, 3], 4), ([5, 1, 9], 3),
                                       ([64, 63, 2], 8), ([13], 5)])
def test_reduce_matches_list_brute_force(numels, nd):
    """Build each rank's full padded gradient from per-tensor lists (pad slots
    hold NaN, which must never be read) and compare every shard slot."""
    rng = np.random.default_rng(sum(numels) + nd)
    per_rank_tensors, full = [], []
    for r in range(nd):
        tensors, buf = [], []
        for n in numels:
            vals = (rng.standard_normal(n) * 1e-2).astype(np.float32)
            tensors.append(vals)
            padded = list(vals)
            while len(padded) % nd:
                padded.append(np.float32(np.nan))
            buf.extend(padded)
        per_rank_tensors.append(tensors)
        full.append(np.array(buf, np.float32))
    for j in range(nd):
        out = oracle.reduce(numels, nd, j, full)
        want = brute_expected(numels, nd, j, per_rank_tensors)
        assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def test_shard_layout_matches_full_layout():
    """A rank-local (shard-layout) input holding exactly the chunk each rank
    sends to rank j gives the same sums as the full layout."""
    numels, nd = [37, 12, 5], 4
    L = oracle.Layout(numels, nd)
    rng = np.random.default_rng(3)
    full = [bf16_bits(rng.standard_normal(L.total_padded) * 1e-3) for _ in range(nd)]
    for j in range(nd):
        chunks = []
        for r in range(nd):
            c = np.zeros(L.S, np.uint16)
            for t in range(len(numels)):
                s = int(L.shard_len[t])
                c[L.shard_off[t]:L.shard_off[t] + s] = \
                    full[r][L.full_off[t] + j * s:L.full_off[t] + (j + 1) * s]
            chunks.append(c)
        a = oracle.reduce(numels, nd, j, full, oracle.GRADS_FULL)
        b = oracle.reduce(numels, nd, j, chunks, oracle.GRADS_SHARD)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_accumulate_is_elementwise_fp32_add():
    a = np.array([1.0, 2.0 ** -24, -3.5, 0.0], np.float32)
    g = np.array([2.0 ** -24, 1.0, 3.5, -0.0], np.float32)
    oracle.accumulate(a, g)
    assert a[0] == np.float32(1.0)                    # tie to even
    assert a[1] == np.float32(1.0)
    assert a[2].view(np.uint32) == 0                   # x + (-x) = +0
    assert a[3].view(np.uint32) == 0                   # +0 + -0 = +0


def test_reduce_values_matches_reduce():
    numels, nd = [50, 3], 5
    L = oracle.Layout(numels, nd)
    rng = np.random.default_rng(5)
    full = [bf16_bits(rng.standard_normal(L.total_padded)) for _ in range(nd)]
    j = 2
    out = oracle.reduce(numels, nd, j, full)
    e = np.arange(L.S)
    t, i = L.locate(e)
    k = j * L.shard_len[t] + i
    valid = k < L.numel[t]
    src = L.full_off[t] + k
    vals = np.stack([f[src[valid]] for f in full], axis=1)
    got = oracle.reduce_values(vals)
    assert np.array_equal(got.view(np.uint32), out[valid].view(np.uint32))
