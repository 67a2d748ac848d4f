"""GPU parity of the span form of the range gather: bf16 work-copy gathers
over short pieces, of at least 64 tiles, starting on a 512-element boundary
(one workgroup per span of tiles stages every rank's run in LDS). Each case
is compared bit for bit with the oracle's gather, and the output buffer's
guard elements before and after the written range must be untouched.

Layouts: parameters of a few to a few thousand elements at N_d = 1, 3, 5
and 8 (pads in many tiles, up to a hundred pieces per tile, rank runs at
every alignment), a total that is not a multiple of 8 (the last source
chunk is read element by element), and layouts with parameters that start
on tile boundaries, whose sub-range gathers begin inside a span, at a
span's start, and end anywhere. Two layouts at N_d = 16 and 64, whose
tiles meet more ranks than a span record holds, check that such layouts
gather by tiles instead (the host tests check which layouts have spans).
"""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp  # noqa: F401
from zero_sharded_mixed_pad_amd import synth

from test_gpu_parity import Mirror, assert_bits, dev, np_of

pytestmark = pytest.mark.gpu

GUARD = 64  # elements before and after the output range (32-byte multiple)
SENTINEL = 0x7fa5  # a bf16 NaN pattern no gather produces from these inputs


def aligned_groups(seed, groups, lo, hi):
    """Random short parameters in groups, each group closed by a filler that
    brings the running total to a multiple of 512: the parameter after each
    filler starts on a tile boundary."""
    rng = np.random.default_rng(seed)
    out, total = [], 0
    for _ in range(groups):
        for n in np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi), int(rng.integers(3, 40))))):
            out.append(int(n))
            total += int(n)
        fill = (-total) % 512
        if fill:
            out.append(fill)
            total += fill
    return out


LAYOUTS = {
    "log_uniform_nd8": (synth.small_tensor_sizes(count=1500, lo=64, hi=16384, seed=11), 8),
    "tiny_nd8": (synth.small_tensor_sizes(count=3000, lo=1, hi=300, seed=12), 8),
    "odd_nd3": (synth.small_tensor_sizes(count=800, lo=10, hi=5000, seed=13), 3),
    "padded_nd16": (synth.small_tensor_sizes(count=1000, lo=17, hi=9000, seed=14), 16),
    "tiny_nd64": (synth.small_tensor_sizes(count=2000, lo=64, hi=700, seed=15), 64),
    "nd1": (synth.small_tensor_sizes(count=3000, lo=10, hi=200, seed=16), 1),
    "ragged_end_nd8": (synth.small_tensor_sizes(count=700, lo=5, hi=2000, seed=17) + [13], 8),
    "aligned_starts_nd8": (aligned_groups(18, 60, 8, 3000), 8),
    "aligned_starts_nd5": (aligned_groups(19, 40, 3, 6000), 5),
}


# layouts without span tables: they take the tile form
TILE_FORM = {"padded_nd16", "tiny_nd64"}


def gather_checked(M, a, b, want):
    """Gather parameters [a, b) of the work copy into a guarded buffer."""
    L = M.L
    cnt = int(L.flat_off[b] - L.flat_off[a])
    buf = torch.full((cnt + 2 * GUARD,), SENTINEL, dtype=torch.int16, device=dev())
    out = buf[GUARD:GUARD + cnt].view(torch.bfloat16)
    M.plan.gather_range(a, b - a, out, "work")
    torch.cuda.synchronize()
    got = np_of(buf.view(torch.bfloat16))
    assert_bits(got[GUARD:GUARD + cnt], want, f"span gather [{a},{b})")
    guard = np.concatenate([got[:GUARD], got[GUARD + cnt:]])
    assert np.all(guard == SENTINEL), f"span gather [{a},{b}) wrote outside its output"


@pytest.mark.parametrize("which", list(LAYOUTS))
def test_span_gather_full_range(which):
    numels, nd = LAYOUTS[which]
    M = Mirror(numels, nd, seed=list(LAYOUTS).index(which))
    L = M.L
    assert L.total_numel >= 64 * 512, "layout too small for the span form"
    want = np.concatenate([oracle.gather(numels, nd, t, M.o_work) for t in range(L.T)])
    gather_checked(M, 0, L.T, want)
    # the master copy (fp32) takes the tile form; it must agree too
    out = torch.empty(L.total_numel, dtype=torch.float32, device=dev())
    M.plan.gather_range(0, L.T, out, "master")
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), M.flat.float()), "gather(partition(x)) != x (master)"


@pytest.mark.parametrize("which", ["aligned_starts_nd8", "aligned_starts_nd5"])
def test_span_gather_aligned_subranges(which):
    numels, nd = LAYOUTS[which]
    M = Mirror(numels, nd, seed=7)
    L = M.L
    per_t = [oracle.gather(numels, nd, t, M.o_work) for t in range(L.T)]
    starts = [t for t in range(L.T) if L.flat_off[t] % 512 == 0 and L.numel[t] > 0]
    assert len(starts) >= 10
    rng = np.random.default_rng(3)
    cases = [(starts[1], L.T), (starts[2], starts[-1])]
    for _ in range(16):
        a = int(rng.choice(starts))
        # at least 64 tiles from a, so the span form is taken
        b_min = int(np.searchsorted(np.asarray(L.flat_off), L.flat_off[a] + 64 * 512))
        if b_min >= L.T:
            continue
        cases.append((a, int(rng.integers(b_min + 1, L.T + 1))))
    for a, b in cases:
        gather_checked(M, a, b, np.concatenate(per_t[a:b]))


def test_span_gather_after_steps():
    """The span gather reads the work copy the fused step wrote."""
    numels, nd = LAYOUTS["log_uniform_nd8"]
    M = Mirror(numels, nd, seed=21)
    for step in (1, 2):
        g = M.grads(torch.bfloat16, f"span{step}")
        M.plan.reduce_adam_step(zsp.ALL_RANKS, [x.to(dev()) for x in g], step=step,
                                lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
        for j in M.ranks:
            M.o_adam(j, M.o_reduce(j, g), step)
    assert M.check_state("steps before span gather") == 0
    want = np.concatenate([oracle.gather(numels, nd, t, M.o_work) for t in range(M.L.T)])
    gather_checked(M, 0, M.L.T, want)
