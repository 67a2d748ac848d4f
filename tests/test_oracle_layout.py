"""Pins for the oracle's layout, copy-in, gather and accounting.

Everything here is checked against something other than the oracle's own
offset arithmetic: a search for the pad, an explicit list-based flatten /
pad / split of every tensor (brute force over every index), the round-trip
property, and the worked example printed on the pages.
"""
import numpy as np
import pytest
import torch

import oracle
from golden_io import read as read_golden


def brute_pad(numel, nd):
    """Smallest p >= 0 with (numel + p) divisible by nd, found by search."""
    p = 0
    while (numel + p) % nd:
        p += 1
    return p


def brute_partition(numels, nd):
    """Flatten, pad and split with Python lists ("The ZeRO-3 Diagram Most
    People Remember Is Wrong", section 2, steps 1-4).

    Each element is labelled (t, k) with k its flat index in tensor t, or
    (t, None) for a pad slot. Returns the full padded concatenation and the
    list of labels each rank stores, tensor after tensor.
    """
    full, shards = [], [[] for _ in range(nd)]
    for t, n in enumerate(numels):
        padded = [(t, k) for k in range(n)]
        while len(padded) % nd:
            padded.append((t, None))
        full.extend(padded)
        s = len(padded) // nd
        for r in range(nd):
            shards[r].extend(padded[r * s:(r + 1) * s])
    return full, shards


def test_pad_closed_form_and_search_agree():
    for nd in range(1, 10):
        for numel in range(0, 65):
            p = oracle.pad(numel, nd)
            assert p == brute_pad(numel, nd)
            assert p == (nd - numel % nd) % nd
            assert 0 <= p < nd and (numel + p) % nd == 0


def _layout_cases():
    cases = [([n], nd) for nd in range(1, 10) for n in range(0, 65)]
    rng = np.random.default_rng(1234)
    for _ in range(60):
        nd = int(rng.integers(1, 10))
        T = int(rng.integers(1, 7))
        numels = [int(x) for x in rng.integers(0, 40, size=T)]
        cases.append((numels, nd))
    cases.append(([1, 1, 1, 1, 1], 8))          # every tensor smaller than N_d
    cases.append(([0, 0, 5, 0], 3))             # empty tensors between others
    cases.append(([97, 89, 83], 7))             # primes
    return cases


@pytest.mark.parametrize("numels,nd", _layout_cases())
def test_layout_matches_brute_force(numels, nd):
    L = oracle.Layout(numels, nd)
    full, shards = brute_partition(numels, nd)
    assert L.total_padded == len(full)
    assert all(len(s) == L.S for s in shards)
    assert L.S * nd == len(full)
    for t, n in enumerate(numels):
        assert L.pad[t] == brute_pad(n, nd)
        assert L.shard_len[t] * nd == n + L.pad[t]
    # Every shard position maps to the label brute force put there.
    for r in range(nd):
        for e in range(L.S):
            tt, ii = L.locate(np.array([e]))
            t, i = int(tt[0]), int(ii[0])
            k = r * int(L.shard_len[t]) + i
            want = shards[r][e]
            assert want[0] == t
            assert want[1] == (k if k < numels[t] else None)
    # Full-layout offsets place padded tensors back to back.
    for t, n in enumerate(numels):
        for k in range(n + int(L.pad[t])):
            assert full[int(L.full_off[t]) + k] == (t, k if k < n else None)
    # Unpadded offsets are the prefix sums of numel.
    assert list(L.flat_off) == list(np.concatenate([[0], np.cumsum(numels)]))


@pytest.mark.parametrize("numels,nd", _layout_cases()[::7])
def test_partition_places_every_element(numels, nd):
    total = int(sum(numels))
    rng = np.random.default_rng(7)
    flat = rng.standard_normal(total).astype(np.float32)
    master, work, m, v = oracle.partition(numels, nd, flat)
    L = oracle.Layout(numels, nd)
    _, shards = brute_partition(numels, nd)
    for r in range(nd):
        for e in range(L.S):
            t, k = shards[r][e]
            got = master[r * L.S + e]
            if k is None:
                assert got.view(np.uint32) == 0          # +0.0 pad
                assert work[r * L.S + e] == 0
            else:
                assert got.view(np.uint32) == flat[L.flat_off[t] + k].view(np.uint32)
    assert not m.view(np.uint32).any() and not v.view(np.uint32).any()


ROUNDTRIP_SHAPES = [
    ([1003, 1000], 4), ([1001 * 7], 4), ([1], 1), ([0], 4), ([3], 8), ([5], 8),
    ([97], 16), ([64, 65, 1, 0, 4096, 11], 8), ([31, 17, 2], 5),
]


@pytest.mark.parametrize("numels,nd", ROUNDTRIP_SHAPES)
def test_roundtrip_fp32_and_bf16(numels, nd):
    """gather(partition(x)) == x, bit for bit: compute sees the full tensor
    exactly as if it had never been sharded ("The ZeRO-3 Diagram Most People
    Remember Is Wrong", section 2, last paragraph)."""
    total = int(sum(numels))
    g = torch.Generator().manual_seed(11)
    x32 = (torch.randn(total, generator=g) * 0.02).numpy().astype(np.float32)
    xbf = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    L = oracle.Layout(numels, nd)
    for flat in (x32, xbf):
        master, work, m, v = oracle.partition(numels, nd, flat)
        for t in range(len(numels)):
            lo, hi = L.flat_off[t], L.flat_off[t + 1]
            back = oracle.gather(numels, nd, t, master)
            want32 = oracle.bf16_to_f32(flat[lo:hi]) if flat.dtype == np.uint16 else flat[lo:hi]
            assert np.array_equal(back.view(np.uint32), want32.view(np.uint32))
            wb = oracle.gather(numels, nd, t, work)
            if flat.dtype == np.uint16:
                assert np.array_equal(wb, flat[lo:hi])
            else:
                ref = torch.from_numpy(flat[lo:hi].copy()).to(torch.bfloat16)
                assert np.array_equal(wb, ref.view(torch.int16).numpy().view(np.uint16))


def test_accounting_worked_example():
    """Equation M_Stage3 and its 7B / 64-GPU example ("ZeRO Stage 3: Parameter
    Partitioning"): 16*7e9/64 bytes = 1.75 GB per GPU."""
    g = read_golden("accounting_7b_n64.txt")
    assert g["psi"] % g["n_d"] == 0
    per_rank = oracle.model_state_bytes(g["psi"] // g["n_d"])
    assert per_rank == g["per_gpu_bytes"]
    assert oracle.model_state_bytes(g["psi"]) == g["total_bytes"]
    assert g["bytes_per_param"] * g["psi"] == g["total_bytes"]


def test_accounting_7b_shaped_model():
    """The 7B-shaped model (32 Llama layers of d=4096, FFN 11008, plus a
    32000x4096 embedding and LM head) at N_d=64: 16*S per rank equals
    16*psi/N_d exactly because no tensor needs padding."""
    d, f, vocab = 4096, 11008, 32000
    layer = [d * d] * 4 + [d * f] * 3 + [d] * 2
    numels = layer * 32 + [vocab * d] * 2
    L = oracle.Layout(numels, 64)
    psi = sum(numels)
    assert psi == 6_738_411_520
    assert L.S == 105_287_680 and L.pad.sum() == 0
    assert oracle.model_state_bytes(L.S) == 16 * psi // 64 == 1_684_602_880
