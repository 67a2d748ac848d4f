"""The C oracle against oracle/brute.py, a second CPU implementation written
differently (lists of indices for the layout, numpy float32 scalars one
operation at a time for the arithmetic, exact rational arithmetic for the
bf16 rounding), bit for bit on tiny inputs. Agreement checks the oracle's
implementation -- slicing and offsets, operation order, no FMA contraction or
excess precision from the compiler -- over several Adam steps, with and
without an accumulated micro-batch, where the other pins bound the result
only to within rounding. The mathematics is pinned separately (closed forms,
bounds, brute force over indices, the pages' worked example)."""
import numpy as np
import pytest

import oracle
from oracle import brute

HP = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8)

LAYOUTS = [
    ([5, 0, 7], 3),
    ([1, 2, 3, 4, 5, 6, 7, 8, 9], 4),
    ([64], 4),
    ([13, 1, 30], 1),
    ([17, 3, 0, 11], 5),
    ([2, 2, 2], 7),
]


@pytest.mark.parametrize("numel,nd", LAYOUTS + [([n], d) for n in range(0, 21) for d in (1, 2, 3, 6)])
def test_layout_tables_agree(numel, nd):
    L = oracle.Layout(numel, nd)
    B = brute.layout(numel, nd)
    assert list(L.pad) == B["pad"]
    assert list(L.shard_len) == B["shard_len"]
    assert list(L.full_off) == B["full_off"]
    assert list(L.shard_off) == B["shard_off"]
    assert list(L.flat_off) == B["flat_off"]
    assert L.S == B["S"]


def test_bf16_rounding_by_value_agrees_with_the_oracle():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x3f808000, 0x3f818000, 0x3f80ffff,
                        0x7f7fffff, 0x7f7f8000, 0x7f7f7fff, 0xff7fffff, 0x00000001,
                        0x00008000, 0x00018000, 0x007fffff, 0x80008001, 0x7f800000,
                        0xff800000, 0x7fc00000, 0x7f800001, 0xffa5a5a5], np.uint32)
    x = np.concatenate([bits, special]).view(np.float32)
    want = oracle.bf16_rne(x)
    got = np.array([brute.bf16(v) for v in x], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), hex(int(got[i])), hex(int(want[i])))
                           for i in bad[:5]]


def _grads(rng, total_padded, nd, special):
    """bf16 gradient buffers (bit patterns) for nd ranks, full padded layout."""
    g = rng.normal(0.0, 1e-2, size=(nd, total_padded)).astype(np.float32)
    if special:
        flat = g.reshape(-1)
        idx = rng.choice(flat.size, size=max(1, flat.size // 8), replace=False)
        flat[idx] = rng.choice(np.array([3e38, -3e38, 1e-39, -1e-42, 65504.0, 1e-30, 0.0,
                                         -0.0], np.float32), size=idx.size)
    return oracle.bf16_rne(g)


def _same_bits(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a.view(np.uint32) == b.view(np.uint32))))


@pytest.mark.parametrize("numel,nd", LAYOUTS)
@pytest.mark.parametrize("special", [False, True])
@pytest.mark.parametrize("with_acc", [False, True])
def test_steps_agree_bit_for_bit(numel, nd, special, with_acc):
    """Copy-in, then four steps of reduce (+ an accumulated earlier
    micro-batch) and Adam, every rank: master, m, v and the bf16 copy equal
    bit for bit after every step (NaN positions compared as NaN)."""
    rng = np.random.default_rng(brute.f32_bits(np.float32(len(numel) + 0.25 * nd)) + special)
    L = oracle.Layout(numel, nd)
    flat = rng.normal(0.0, 0.02, size=max(L.total_numel, 1)).astype(np.float32)
    master, work, m, v = oracle.partition(numel, nd, flat)
    B = brute.Model(numel, nd, flat)
    S = L.S
    with np.errstate(all="ignore"):
        for j in range(nd):
            assert _same_bits(master[j * S:(j + 1) * S], B.master[j])
            assert list(work[j * S:(j + 1) * S]) == B.work[j]
        for step in range(1, 5):
            g = _grads(rng, max(L.total_padded, 1), nd, special)
            acc_o = acc_b = None
            if with_acc:
                g0 = _grads(rng, max(L.total_padded, 1), nd, special)
                gw0 = [brute.bf16_widen_array(g0[r]) for r in range(nd)]
                acc_o = [oracle.reduce(numel, nd, j, list(g0)) for j in range(nd)]
                acc_b = [[x if x is not None else np.float32(0.0) for x in B.reduce(gw0, j)]
                         for j in range(nd)]
                for j in range(nd):
                    assert _same_bits(acc_o[j], acc_b[j]), f"reduce, rank {j}, step {step}"
            for j in range(nd):
                red = oracle.reduce(numel, nd, j, list(g))
                if with_acc:
                    oracle.accumulate(acc_o[j], red)
                    red = acc_o[j]
                sl = slice(j * S, (j + 1) * S)
                mj, mmj, vj, wj = master[sl].copy(), m[sl].copy(), v[sl].copy(), work[sl].copy()
                oracle.adam(numel, nd, j, mj, mmj, vj, wj, red, HP["lr"], HP["b1"], HP["b2"],
                            HP["eps"], step)
                master[sl], m[sl], v[sl], work[sl] = mj, mmj, vj, wj
            gw = [brute.bf16_widen_array(g[r]) for r in range(nd)]
            B.step(gw, HP["lr"], HP["b1"], HP["b2"], HP["eps"], step, acc=acc_b)
            for j in range(nd):
                sl = slice(j * S, (j + 1) * S)
                what = f"step {step}, rank {j}"
                assert _same_bits(master[sl], B.master[j]), f"master, {what}"
                assert _same_bits(m[sl], B.m[j]), f"m, {what}"
                assert _same_bits(v[sl], B.v[j]), f"v, {what}"
                wo = np.asarray(work[sl], np.uint16)
                wb = np.asarray(B.work[j], np.uint16)
                nan_o = np.isnan(oracle.bf16_to_f32(wo))
                nan_b = np.isnan(oracle.bf16_to_f32(wb))
                assert np.array_equal(nan_o, nan_b) and np.array_equal(wo[~nan_o], wb[~nan_b]), \
                    f"work, {what}"


try:
    from hypothesis import given, settings, strategies as st
except ImportError:  # the property test below needs hypothesis
    given = None

if given is not None:
    @settings(max_examples=300, deadline=None)
    @given(numel=st.lists(st.integers(0, 300), min_size=1, max_size=12),
           nd=st.integers(1, 17))
    def test_layout_tables_agree_on_random_lists(numel, nd):
        """Random parameter lists: the oracle's tables equal those read off the
        padded, sliced index lists, and every owner position maps to the
        element the slices give it."""
        L = oracle.Layout(numel, nd)
        B = brute.layout(numel, nd)
        assert (list(L.pad), list(L.shard_len), list(L.full_off), list(L.shard_off),
                list(L.flat_off), L.S) == (B["pad"], B["shard_len"], B["full_off"],
                                           B["shard_off"], B["flat_off"], B["S"])
        own = brute.owners(numel, nd)
        for j in range(nd):
            assert len(own[j]) == L.S
            for k, o in enumerate(own[j]):
                t, i = L.locate(k)
                elem = int(j * L.shard_len[t] + i)     # element of parameter t held there
                assert o == (None if elem >= numel[t] else (int(t), elem))
