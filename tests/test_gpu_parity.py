"""GPU parity: every libzsp entry point against the CPU oracle, element by
element, on seeded inputs small enough for the oracle but spanning many
512-element tiles, ragged tails, padded tensors, empty tensors and tensors
smaller than N_d.

Bar: layout, copy-in, reduce, accumulation and gather bit-exact; Adam
master, m and v within 2 ulp or 1e-6 relative (the kernels are expected to
be bit-exact and the tests report the largest distance); the bf16 working
copy within 1 bf16 ulp.
"""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_pad_amd as zsp
from zero_sharded_mixed_pad_amd import synth

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def dev():
    return torch.device("cuda")


def np_of(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def torch_of(a, device):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(a.copy()).to(device)


def ordered(bits, width):
    k = bits.astype(np.int64)
    sign = 1 << (width - 1)
    return np.where(k & sign, -(k & (sign - 1)), k)


def assert_f32_close(got, want, what):
    g, w = got.view(np.uint32), want.view(np.uint32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    ok = ~wn
    ulp = np.abs(ordered(g[ok], 32) - ordered(w[ok], 32))
    with np.errstate(invalid="ignore"):   # inf - inf: the ulp test decides those
        rel = (np.abs(got[ok].astype(np.float64) - want[ok])
               <= 1e-6 * np.abs(want[ok].astype(np.float64)))
    bad = ~((ulp <= 2) | rel)
    assert not bad.any(), f"{what}: {bad.sum()} elements off, max ulp {ulp.max()}"
    return int(ulp.max()) if ulp.size else 0


def assert_bf16_close(got, want, what):
    gn = np.isnan(oracle.bf16_to_f32(got))
    wn = np.isnan(oracle.bf16_to_f32(want))
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    ulp = np.abs(ordered(got[~wn], 16) - ordered(want[~wn], 16))
    assert ulp.size == 0 or ulp.max() <= 1, f"{what}: max bf16 ulp {ulp.max()}"
    return int(ulp.max()) if ulp.size else 0


def assert_bits(got, want, what):
    assert got.dtype == want.dtype
    if not np.array_equal(got.view(np.uint8), want.view(np.uint8)):
        diff = np.flatnonzero(got.view(np.uint32 if got.itemsize == 4 else np.uint16) !=
                              want.view(np.uint32 if want.itemsize == 4 else np.uint16))
        raise AssertionError(f"{what}: {diff.size} elements differ, first at {diff[:5]}")


class Mirror:
    """A plan with state on the GPU and the same state held by the oracle."""

    def __init__(self, numels, nd, pdtype=torch.bfloat16, seed=0, rank_local=None,
                 with_acc=True):
        self.numels, self.nd = list(numels), nd
        self.L = oracle.Layout(numels, nd)
        self.rank_local = rank_local
        self.ranks = list(range(nd)) if rank_local is None else [rank_local]
        self.flat = synth.normal(self.L.total_numel, 0.02, pdtype,
                                 synth.derive_seed("parity", seed, "params"))
        lo, hi = (0, nd) if rank_local is None else (rank_local, rank_local + 1)
        self.o_master, self.o_work, self.o_m, self.o_v = oracle.partition(
            numels, nd, np_of(self.flat), lo, hi)
        n = (hi - lo) * self.L.S
        self.o_acc = np.zeros(n, np.float32)
        self.plan = zsp.partition(numels, nd)
        alloc = max(n, 64)
        d = dev()
        self.g_master = torch.empty(alloc, dtype=torch.float32, device=d)
        self.g_m = torch.empty(alloc, dtype=torch.float32, device=d)
        self.g_v = torch.empty(alloc, dtype=torch.float32, device=d)
        self.g_work = torch.empty(alloc, dtype=torch.bfloat16, device=d)
        self.g_acc = torch.zeros(alloc, dtype=torch.float32, device=d) if with_acc else None
        self.n = n
        self.plan.bind_state(zsp.ALL_RANKS if rank_local is None else rank_local, self.g_master,
                             self.g_m, self.g_v, self.g_work, self.g_acc)
        self.plan.load_params(self.flat.to(d))

    # ---- inputs -----------------------------------------------------------
    def grads(self, dtype, tag, layout="full", poison=True, sigma=1e-2):
        """nd gradient buffers (CPU tensors); pad slots of full-layout buffers
        hold NaN so that reading one would show."""
        L = self.L
        if layout == "full":
            size = L.total_padded
        else:
            size = L.S if self.rank_local is not None else self.nd * L.S
        out = []
        for r in range(self.nd):
            g = synth.normal(size, sigma, dtype, synth.derive_seed("parity", tag, r))
            if poison and layout == "full":
                for t in range(L.T):
                    a, b = int(L.full_off[t] + L.numel[t]), int(L.full_off[t + 1])
                    g[a:b] = float("nan")
            out.append(g)
        return out

    # ---- oracle side ------------------------------------------------------
    def o_slice(self, j):
        base = 0 if self.rank_local is not None else j * self.L.S
        return slice(base, base + self.L.S)

    def o_reduce(self, j, grads, layout="full"):
        gnp = [np_of(g) for g in grads]
        if layout == "full":
            return oracle.reduce(self.numels, self.nd, j, gnp, oracle.GRADS_FULL)
        if self.rank_local is None:
            gnp = [g[j * self.L.S:(j + 1) * self.L.S] for g in gnp]
        return oracle.reduce(self.numels, self.nd, j, gnp, oracle.GRADS_SHARD)

    def o_adam(self, j, g, step, hp=HP):
        sl = self.o_slice(j)
        oracle.adam(self.numels, self.nd, j, self.o_master[sl], self.o_m[sl], self.o_v[sl],
                    self.o_work[sl], g, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], step)

    # ---- compare ------------------------------------------------------------
    def check_state(self, what, exact=False):
        torch.cuda.synchronize()
        n = self.n
        got = [np_of(x[:n]) for x in (self.g_master, self.g_m, self.g_v, self.g_work)]
        want = [self.o_master, self.o_m, self.o_v, self.o_work]
        if exact:
            for name, g, w in zip(("master", "m", "v", "work"), got, want):
                assert_bits(g, w, f"{what}/{name}")
            return 0
        u = [assert_f32_close(g, w, f"{what}/{name}")
             for name, g, w in zip(("master", "m", "v"), got[:3], want[:3])]
        u.append(assert_bf16_close(got[3], want[3], f"{what}/work"))
        return max(u)

    def check_acc(self, what):
        torch.cuda.synchronize()
        assert_bits(np_of(self.g_acc[:self.n]), self.o_acc, what)


CASES = [
    ([1003, 64, 5, 0, 3 * 4096 + 1], 4),
    ([1000 * 1003], 4),
    ([1001 * 1003], 4),
    ([4096 * 3, 11008 * 2, 4096, 4096], 8),
    ([1, 2, 3, 5, 7, 11, 13, 17, 19, 23, 29], 8),
    ([511 * 8, 512 * 8, 513 * 8, 8 * 8 * 64 + 3], 8),
    ([97, 0, 0, 12345], 16),
    ([3] * 40 + [1000], 64),
    ([77777], 1),
    ([300, 7, 5000], 256),
    ([1003, 64, 5, 0, 3 * 4096 + 1], 40),   # ranks in batches of 16 with a partial batch
    ([300 * 1001, 7, 200 * 513 + 3, 65536], 4),   # long pieces, unaligned parameter starts
    ([97, 12345, 7, 2048], 100),
    (synth.small_tensor_sizes(count=300, lo=8, hi=3000, seed=5), 8),
]


@pytest.mark.parametrize("numels,nd", CASES)
@pytest.mark.parametrize("pdtype", [torch.bfloat16, torch.float32])
def test_copyin_bit_exact(numels, nd, pdtype):
    M = Mirror(numels, nd, pdtype)
    M.check_state("copy-in", exact=True)


@pytest.mark.parametrize("numels,nd", CASES)
def test_gather_roundtrip_and_oracle(numels, nd):
    for pdtype in (torch.bfloat16, torch.float32):
        M = Mirror(numels, nd, pdtype)
        d = dev()
        L = M.L
        allw = torch.empty(max(L.total_numel, 8), dtype=torch.bfloat16, device=d)
        allm = torch.empty(max(L.total_numel, 8), dtype=torch.float32, device=d)
        M.plan.gather_range(0, L.T, allw, "work")
        M.plan.gather_range(0, L.T, allm, "master")
        torch.cuda.synchronize()
        flat32 = M.flat.float()
        assert torch.equal(allm[:L.total_numel].cpu(), flat32), "gather(partition(x)) != x"
        want_w = np.concatenate([oracle.gather(numels, nd, t, M.o_work) for t in range(L.T)])
        assert_bits(np_of(allw[:L.total_numel]), want_w, "gather_range/work")
        # single-tensor gathers into fresh buffers
        for t in range(L.T):
            nt = int(L.numel[t])
            out = torch.full((max(nt, 8),), float("nan"), dtype=torch.bfloat16, device=d)
            M.plan.gather(t, out, "work")
            torch.cuda.synchronize()
            assert_bits(np_of(out[:nt]), oracle.gather(numels, nd, t, M.o_work), f"gather {t}")


# Short pieces take the gather's short-piece form; long ones its default form,
# whose launches starting on a 512-element boundary look up one delta per tile.
SUBRANGE_LAYOUTS = {
    "short": (synth.small_tensor_sizes(count=200, lo=5, hi=2000, seed=9), 8),
    "long": ([512 * 300, 4096 * 37 + 5, 100003, 77, 262144 + 13, 512 * 64, 9000], 8),
    # short pieces with a tile-aligned second parameter (per-tile pair records)
    "short_aligned": ([512 * 3, 8000, 7777, 15000, 640, 20480, 3, 15000, 9, 4096], 8),
}


@pytest.mark.parametrize("which", list(SUBRANGE_LAYOUTS))
def test_gather_range_subranges(which):
    numels, nd = SUBRANGE_LAYOUTS[which]
    M = Mirror(numels, nd)
    L = M.L
    rng = np.random.default_rng(0)
    d = dev()
    ranges = [(0, L.T), (1, L.T), (1, 2)]
    for _ in range(20):
        a = int(rng.integers(0, L.T))
        ranges.append((a, int(rng.integers(a + 1, L.T + 1))))
    for a, b in ranges:
        cnt = int(L.flat_off[b] - L.flat_off[a])
        out = torch.empty(max(cnt, 8), dtype=torch.bfloat16, device=d)
        M.plan.gather_range(a, b - a, out, "work")
        torch.cuda.synchronize()
        want = np.concatenate([oracle.gather(numels, nd, t, M.o_work) for t in range(a, b)])
        assert_bits(np_of(out[:cnt]), want, f"gather_range[{a},{b})")


@pytest.mark.parametrize("numels,nd", CASES)
@pytest.mark.parametrize("gdtype", [torch.bfloat16, torch.float32])
def test_fused_steps_match_oracle(numels, nd, gdtype):
    M = Mirror(numels, nd, torch.float32 if gdtype == torch.float32 else torch.bfloat16)
    worst = 0
    for step in (1, 2, 3):
        grads = M.grads(gdtype, ("fused", step))
        M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(dev()) for g in grads], step=step, **HP)
        for j in M.ranks:
            M.o_adam(j, M.o_reduce(j, grads), step)
        worst = max(worst, M.check_state(f"step {step}"))
    assert worst == 0, f"not bit-exact: max ulp {worst}"


@pytest.mark.parametrize("numels,nd", CASES[:6])
def test_reduce_accumulate_and_adam_from_acc(numels, nd):
    M = Mirror(numels, nd)
    d = dev()
    g0 = M.grads(torch.bfloat16, "acc0")
    M.plan.reduce_shard(zsp.ALL_RANKS, [g.to(d) for g in g0], accumulate=False)
    for j in M.ranks:
        M.o_acc[M.o_slice(j)] = M.o_reduce(j, g0)
    M.check_acc("reduce set")
    for k in (1, 2):
        gk = M.grads(torch.bfloat16, ("acc", k))
        M.plan.reduce_shard(zsp.ALL_RANKS, [g.to(d) for g in gk], accumulate=True)
        for j in M.ranks:
            oracle.accumulate(M.o_acc[M.o_slice(j)], M.o_reduce(j, gk))
        M.check_acc(f"reduce accumulate {k}")
    M.plan.adam_step(zsp.ALL_RANKS, step=1, **HP)
    for j in M.ranks:
        M.o_adam(j, M.o_acc[M.o_slice(j)].copy(), 1)
    assert M.check_state("adam from acc") == 0


@pytest.mark.parametrize("numels,nd", CASES[:6])
def test_fused_use_acc_equals_accumulate_then_adam(numels, nd):
    M = Mirror(numels, nd)
    d = dev()
    g0 = M.grads(torch.bfloat16, "ua0")
    M.plan.reduce_shard(zsp.ALL_RANKS, [g.to(d) for g in g0])
    for j in M.ranks:
        M.o_acc[M.o_slice(j)] = M.o_reduce(j, g0)
    g1 = M.grads(torch.bfloat16, "ua1")
    M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(d) for g in g1], step=1, use_acc=True, **HP)
    for j in M.ranks:
        acc = M.o_acc[M.o_slice(j)].copy()
        oracle.accumulate(acc, M.o_reduce(j, g1))
        M.o_adam(j, acc, 1)
    assert M.check_state("fused use_acc") == 0
    M.check_acc("acc untouched by fused step")


def test_single_rank_calls_touch_only_that_rank():
    numels, nd = [1003, 64, 5, 4097], 4
    M = Mirror(numels, nd)
    d = dev()
    for j in (2, 0, 3):
        grads = M.grads(torch.bfloat16, ("one", j))
        M.plan.reduce_adam_step(j, [g.to(d) for g in grads], step=1, **HP)
        M.o_adam(j, M.o_reduce(j, grads), 1)
        assert M.check_state(f"rank {j}") == 0
        M.plan.reduce_shard(j, [g.to(d) for g in grads])
        M.o_acc[M.o_slice(j)] = M.o_reduce(j, grads)
        M.check_acc(f"reduce rank {j}")


@pytest.mark.parametrize("layout", ["shard", "full"])
def test_rank_local_binding(layout):
    numels, nd = [4096 * 5 + 3, 64, 1, 11008 * 2], 16
    for j in (0, 7, 15):
        M = Mirror(numels, nd, rank_local=j)
        M.check_state("rank-local copy-in", exact=True)
        for step in (1, 2):
            grads = M.grads(torch.bfloat16, ("local", j, step), layout=layout)
            M.plan.reduce_adam_step(j, [g.to(dev()) for g in grads], step=step, layout=layout,
                                    **HP)
            M.o_adam(j, M.o_reduce(j, grads, layout), step)
            assert M.check_state(f"rank-local {j} step {step}") == 0
        with pytest.raises(zsp.ZspError) as e:
            M.plan.reduce_adam_step((j + 1) % nd, [g.to(dev()) for g in grads], step=3,
                                    layout=layout, **HP)
        assert e.value.status == zsp.binding.ESTATE
        out = torch.empty(64, dtype=torch.bfloat16, device=dev())
        with pytest.raises(zsp.ZspError) as e:
            M.plan.gather(1, out)
        assert e.value.status == zsp.binding.ESTATE


def test_shard_layout_all_ranks():
    numels, nd = [1003, 64, 5, 3 * 4096 + 1], 4
    M = Mirror(numels, nd)
    grads = M.grads(torch.bfloat16, "shard-all", layout="shard")
    M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(dev()) for g in grads], step=1, layout="shard",
                            **HP)
    for j in M.ranks:
        M.o_adam(j, M.o_reduce(j, grads, "shard"), 1)
    assert M.check_state("shard layout, all ranks") == 0


def test_deterministic_repeat():
    numels, nd = [4096 * 7 + 5, 333], 8
    d = dev()
    res = []
    grads = None
    for _ in range(2):
        M = Mirror(numels, nd)
        grads = grads or M.grads(torch.bfloat16, "det")
        M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(d) for g in grads], step=1, **HP)
        torch.cuda.synchronize()
        res.append([np_of(x) for x in (M.g_master, M.g_m, M.g_v, M.g_work)])
    for a, b in zip(*res):
        assert_bits(a, b, "repeat")


def test_special_values():
    """Zero, subnormal, huge, infinite and NaN gradients follow the oracle."""
    numels, nd = [4096], 4
    M = Mirror(numels, nd, torch.float32)
    L = M.L
    specials = np.array([0.0, -0.0, 1e-40, -1e-42, 3e38, -3e38, np.inf, -np.inf, np.nan,
                         1e-20, 65504.0, 1.0], np.float32)
    grads = []
    for r in range(nd):
        g = np.resize(np.roll(specials, r), L.total_padded).astype(np.float32)
        grads.append(torch.from_numpy(g))
    M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(dev()) for g in grads], step=1, **HP)
    for j in M.ranks:
        M.o_adam(j, M.o_reduce(j, grads), 1)
    assert M.check_state("special values") == 0
    # NaN results of the arithmetic: positions are compared above; report
    # how their bit patterns compare
    got = np_of(M.g_master[:M.n]).view(np.uint32)
    want = M.o_master.view(np.uint32)
    nan = np.isnan(M.o_master)
    pairs = sorted(set(zip(got[nan].tolist(), want[nan].tolist())))
    print(f"[special values] {int(nan.sum())} NaN results; (gpu, oracle) bit pairs: "
          f"{[(hex(a), hex(b)) for a, b in pairs[:8]]}", flush=True)


# fp32 bit patterns of every kind of special value: NaNs (quiet and
# signalling, both signs, payload bits high and low), infinities, signed
# zeros, subnormals, rounding ties to both sides, the largest finite values
# and values that round up to infinity.
SPECIAL_F32 = np.array([
    0x7fc00000, 0xffc00000, 0x7f800001, 0xff800001, 0x7fa00000, 0x7fc12345, 0xffe54321,
    0x7fbfffff, 0xffffffff, 0x7ff0000f, 0x7f800000, 0xff800000, 0x00000000, 0x80000000,
    0x00000001, 0x807fffff, 0x00008000, 0x00018000, 0x3f808000, 0x3f818000, 0x3f80ffff,
    0x7f7fffff, 0xff7fffff, 0x7f7f8000, 0x7f7f7fff, 0x3f7fffff, 0x33800000, 0x00400000,
    0x3f800000, 0xbf800000], np.uint32)


def test_copyin_cast_special_values():
    """fp32 parameters holding the special values above go through the
    copy-in: the master keeps their bits and the bf16 working copy equals the
    oracle's cast bit for bit, NaN payloads and signs included (the cast
    keeps a NaN's sign and leading payload bits and sets its quiet bit)."""
    numels, nd = [SPECIAL_F32.size * 37 + 3, 11], 4
    total = sum(numels)
    flat = np.resize(SPECIAL_F32, total).astype(np.uint32).view(np.float32)
    o_master, o_work, _m, _v = oracle.partition(numels, nd, flat)
    plan = zsp.partition(numels, nd)
    d = dev()
    n = nd * plan.S
    st = [torch.empty(n, dtype=torch.float32, device=d) for _ in range(3)]
    st.append(torch.empty(n, dtype=torch.bfloat16, device=d))
    plan.bind_state(zsp.ALL_RANKS, *st)
    plan.load_params(torch.from_numpy(flat.copy()).to(d))
    torch.cuda.synchronize()
    assert_bits(np_of(st[0]), o_master, "copy-in master (special values)")
    assert_bits(np_of(st[3]), o_work, "copy-in work (special values)")
    # and back through the fp32 gather: every bit pattern comes back
    out = torch.empty(total, dtype=torch.float32, device=d)
    plan.gather_range(0, len(numels), out, "master")
    torch.cuda.synchronize()
    assert_bits(np_of(out), flat.copy(), "gather of special values")
    plan.destroy()


def test_gpu_argument_errors():
    numels, nd = [1003, 64], 4
    M = Mirror(numels, nd)
    d = dev()
    grads = [g.to(d) for g in M.grads(torch.bfloat16, "err")]
    with pytest.raises(zsp.ZspError) as e:
        M.plan.reduce_adam_step(4, grads, step=1, **HP)
    assert e.value.status == zsp.binding.EINVAL
    with pytest.raises(zsp.ZspError) as e:
        M.plan.reduce_adam_step(zsp.ALL_RANKS, grads, step=0, **HP)
    assert e.value.status == zsp.binding.EINVAL
    big = torch.empty(M.L.total_padded + 8, dtype=torch.bfloat16, device=d)
    with pytest.raises(zsp.ZspError) as e:
        M.plan.reduce_adam_step(zsp.ALL_RANKS, [big[1:]] + grads[1:], step=1, **HP)
    assert e.value.status == zsp.binding.EINVAL
    with pytest.raises(ValueError):
        M.plan.reduce_adam_step(zsp.ALL_RANKS, grads[:3], step=1, **HP)
    with pytest.raises(zsp.ZspError) as e:
        M.plan.gather_range(1, 2, torch.empty(2000, dtype=torch.bfloat16, device=d))
    assert e.value.status == zsp.binding.ERANGE
    N = Mirror(numels, nd, with_acc=False)
    with pytest.raises(zsp.ZspError) as e:
        N.plan.adam_step(zsp.ALL_RANKS, step=1, **HP)
    assert e.value.status == zsp.binding.ESTATE
    with pytest.raises(zsp.ZspError) as e:
        N.plan.reduce_adam_step(zsp.ALL_RANKS, grads, step=1, use_acc=True, **HP)
    assert e.value.status == zsp.binding.ESTATE
    # the failed calls enqueued nothing: state still equals the copy-in
    N.check_state("after rejected calls", exact=True)


def test_all_empty_plan(tmp_path):
    """Every parameter empty (S = 0): each entry point succeeds and touches
    nothing; a checkpoint of the empty state round-trips."""
    numels, nd = [0, 0, 0], 4
    plan = zsp.partition(numels, nd)
    assert plan.S == 0 and plan.total_padded == 0 and plan.total_numel == 0
    d = dev()
    st = [torch.full((64,), 7.0, dtype=torch.float32, device=d) for _ in range(3)]
    st.append(torch.full((64,), 7.0, dtype=torch.bfloat16, device=d))
    acc = torch.full((64,), 7.0, dtype=torch.float32, device=d)
    plan.bind_state(zsp.ALL_RANKS, *st, acc)
    plan.load_params(torch.zeros(8, dtype=torch.bfloat16, device=d))
    grads = [torch.zeros(8, dtype=torch.bfloat16, device=d) for _ in range(nd)]
    plan.reduce_adam_step(zsp.ALL_RANKS, grads, step=1, **HP)
    plan.reduce_shard(zsp.ALL_RANKS, grads, accumulate=True)
    plan.adam_step(zsp.ALL_RANKS, step=2, **HP)
    out = torch.full((8,), 3.0, dtype=torch.bfloat16, device=d)
    plan.gather_range(0, 3, out, "work")
    plan.gather(1, out, "work")
    s = zsp.Schedule(plan, [(0, 2), (2, 1)], [0, 1, 1, 0], 1)
    arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=d)
    s.bind(arena, torch.cuda.Stream())
    for p in range(4):
        views = s.acquire(p)
        assert all(v.numel() == 0 for v in views)
        s.release(p)
    s.destroy()
    plan.checkpoint_save(zsp.ALL_RANKS, str(tmp_path), 5)
    assert plan.checkpoint_load(zsp.ALL_RANKS, str(tmp_path)) == 5
    other = zsp.partition(numels, 2)
    st2 = [torch.zeros(64, dtype=torch.float32, device=d) for _ in range(3)]
    st2.append(torch.zeros(64, dtype=torch.bfloat16, device=d))
    other.bind_state(zsp.ALL_RANKS, *st2)
    assert other.checkpoint_load(zsp.ALL_RANKS, str(tmp_path)) == 5   # reshard 4 -> 2
    torch.cuda.synchronize()
    for x in st + [acc]:
        assert torch.all(x.float() == 7.0)
    assert torch.all(out.float() == 3.0)
    plan.destroy()
    other.destroy()


# Layouts for the batched multi-piece path of short-piece launches (up to 16
# ranks, whole tiles): quads crossing into the next piece (two gradient
# vectors), quads crossing a pad boundary, quads meeting three pieces
# (slices under 4 elements), a crossing at the start of a rank's region whose
# next piece's gradient starts within 3 elements of the buffer's start, and
# one near the buffer's end; every piece boundary offset mod 4 occurs.
MULTI_PIECE = {
    "tiny_first": ([1, 1, 2, 3] + [37 + 11 * i for i in range(60)] + [5], 8),
    # s_0 = 2 and S = 3 mod 4: the quad that starts 3 elements before rank
    # 1's region crosses into that rank's slice of parameter 0, whose
    # gradient starts at element 2 of the buffer
    "region_start": ([16] + [37 + 11 * i for i in range(60)] + [25], 8),
    "tiny_last": ([700 + 13 * i for i in range(50)] + [3, 13], 8),
    "boundaries_mod4": ([4 * k + r for k in range(30, 70) for r in range(4)], 5),
    "sixteen": (synth.small_tensor_sizes(count=250, lo=2, hi=4000, seed=31), 16),
    "eight_small": (synth.small_tensor_sizes(count=400, lo=1, hi=900, seed=32), 8),
}


@pytest.mark.parametrize("which", list(MULTI_PIECE))
@pytest.mark.parametrize("layout", ["full", "shard"])
def test_multi_piece_quads_every_op(which, layout):
    numels, nd = MULTI_PIECE[which]
    print(f"\n[multi-piece quads] {which}, {layout} layout", flush=True)
    M = Mirror(numels, nd)
    d = dev()
    g0 = M.grads(torch.bfloat16, ("mp0", which), layout=layout)
    M.plan.reduce_shard(zsp.ALL_RANKS, [g.to(d) for g in g0], layout=layout)
    for j in M.ranks:
        M.o_acc[M.o_slice(j)] = M.o_reduce(j, g0, layout)
    M.check_acc("reduce set")
    g1 = M.grads(torch.bfloat16, ("mp1", which), layout=layout)
    M.plan.reduce_shard(zsp.ALL_RANKS, [g.to(d) for g in g1], layout=layout, accumulate=True)
    for j in M.ranks:
        oracle.accumulate(M.o_acc[M.o_slice(j)], M.o_reduce(j, g1, layout))
    M.check_acc("reduce accumulate")
    g2 = M.grads(torch.bfloat16, ("mp2", which), layout=layout)
    M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(d) for g in g2], step=1, layout=layout,
                            use_acc=True, **HP)
    for j in M.ranks:
        acc = M.o_acc[M.o_slice(j)].copy()
        oracle.accumulate(acc, M.o_reduce(j, g2, layout))
        M.o_adam(j, acc, 1)
    assert M.check_state("fused with the accumulator") == 0
    for step in (2, 3):
        gs = M.grads(torch.float32, ("mp", which, step), layout=layout)
        M.plan.reduce_adam_step(zsp.ALL_RANKS, [g.to(d) for g in gs], step=step, layout=layout,
                                **HP)
        for j in M.ranks:
            M.o_adam(j, M.o_reduce(j, gs, layout), step)
        assert M.check_state(f"fused step {step} (fp32 gradients)") == 0
    M.plan.adam_step(zsp.ALL_RANKS, step=4, **HP)
    for j in M.ranks:
        M.o_adam(j, M.o_acc[M.o_slice(j)].copy(), 4)
    assert M.check_state("adam from the accumulator") == 0
