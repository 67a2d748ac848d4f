"""Pins for the oracle's Adam step and bf16 working-copy refresh.

The pages name Adam with fp32 master weights and fp32 moments but do not
print the update; the oracle follows Kingma & Ba, Algorithm 1. It is pinned
here by closed forms of that algorithm (first step from zero moments; a
constant gradient, for which the bias-corrected moments are exactly g and
g^2 at every step; a zero gradient; beta1 = beta2 = 0), by the unrolled
form of the moment recursions evaluated in float64 within a derived
rounding bound, by the step-size bound of Kingma & Ba section 2.1, and by
torch's own round-to-nearest-even bf16 cast.
"""
import numpy as np
import pytest
import torch

import oracle

U = 2.0 ** -24
LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def f64(x):
    return float(np.float32(x))


def torch_bf16_bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fresh(n, p0=0.0):
    return (np.full(n, p0, np.float32), np.zeros(n, np.float32),
            np.zeros(n, np.float32), np.zeros(n, np.uint16))


def grads(n, seed, scale=1e-2):
    g = np.random.default_rng(seed).standard_normal(n) * scale
    return g.astype(np.float32)


def test_first_step_closed_form():
    """From m = v = 0: m1 = (1-b1) g, v1 = (1-b2) g^2, and the step is
    lr * g / (|g| + eps) (bias correction undoes the (1-b) factors)."""
    n = 20000
    g = grads(n, 0)
    p, m, v, w = fresh(n)
    oracle.adam_elems(p, m, v, w, g, LR, B1, B2, EPS, 1)
    omb1 = np.float32(1.0) - np.float32(B1)
    omb2 = np.float32(1.0) - np.float32(B2)
    assert np.array_equal(m, (omb1 * g).astype(np.float32))
    assert np.array_equal(v, (omb2 * (g * g)).astype(np.float32))
    g64 = g.astype(np.float64)
    step = f64(LR) * g64 / (np.abs(g64) + f64(EPS))
    rel = np.abs(-p.astype(np.float64) - step) / np.abs(step)
    assert rel.max() <= 1e-6


def test_first_step_from_nonzero_master():
    n = 5000
    rng = np.random.default_rng(1)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = grads(n, 2)
    p, m, v, w = fresh(n)
    p[:] = p0
    oracle.adam_elems(p, m, v, w, g, LR, B1, B2, EPS, 1)
    g64 = g.astype(np.float64)
    want = p0.astype(np.float64) - f64(LR) * g64 / (np.abs(g64) + f64(EPS))
    # one rounding of the result plus ~8u relative in the step
    tol = np.spacing(np.abs(p).astype(np.float32)).astype(np.float64) + 1e-6 * f64(LR)
    assert np.all(np.abs(p.astype(np.float64) - want) <= tol)


@pytest.mark.parametrize("steps", [1, 2, 5, 30])
def test_constant_gradient_closed_form(steps):
    """With g fixed, m_t = g (1-b1^t) and v_t = g^2 (1-b2^t), so after bias
    correction every step is lr * g / (|g| + eps): p_t = p_0 - t * that.
    An off-by-one or missing bias correction breaks this at t = 1 or 2."""
    n = 4096
    g = grads(n, 3)
    p, m, v, w = fresh(n)
    for t in range(1, steps + 1):
        oracle.adam_elems(p, m, v, w, g, LR, B1, B2, EPS, t)
    g64 = g.astype(np.float64)
    want = -steps * f64(LR) * g64 / (np.abs(g64) + f64(EPS))
    rel = np.abs(p.astype(np.float64) - want) / np.abs(want)
    assert rel.max() <= 2e-6 * steps


def test_zero_gradient_leaves_parameter():
    n = 1000
    rng = np.random.default_rng(4)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p, m, v, w = fresh(n)
    p[:] = p0
    for t in range(1, 4):
        oracle.adam_elems(p, m, v, w, np.zeros(n, np.float32), LR, B1, B2, EPS, t)
    assert np.array_equal(p, p0)
    assert not m.any() and not v.any()
    assert np.array_equal(w, torch_bf16_bits(p0))


def test_no_momentum_is_normalised_step():
    """b1 = b2 = 0: m = g, v = g^2, no bias correction, so each step is
    lr * g / (|g| + eps) whatever came before."""
    n = 3000
    p, m, v, w = fresh(n)
    for t in range(1, 5):
        g = grads(n, 10 + t)
        p[:] = 0.0
        oracle.adam_elems(p, m, v, w, g, LR, 0.0, 0.0, EPS, t)
        g64 = g.astype(np.float64)
        want = -f64(LR) * g64 / (np.abs(g64) + f64(EPS))
        assert (np.abs(p.astype(np.float64) - want) / np.abs(want)).max() <= 1e-6


def unrolled_reference(p0, gs, lr, b1, b2, eps):
    """Float64 Adam from the unrolled moments:
       m_t = sum_k (1-b1) b1^(t-k) g_k ,  v_t = sum_k (1-b2) b2^(t-k) g_k^2
    plus an error bound for an fp32 evaluation of the recursive form.
    Returns the parameter after every step and the bound on each."""
    b1, b2, lr, eps = f64(b1), f64(b2), f64(lr), f64(eps)
    omb1, omb2 = f64(np.float32(1) - np.float32(b1)), f64(np.float32(1) - np.float32(b2))
    T = len(gs)
    G = np.stack([g.astype(np.float64) for g in gs])
    p = p0.astype(np.float64).copy()
    err_p = np.zeros_like(p)
    err_m = np.zeros_like(p)       # bound on |m_fp32 - m| (absolute)
    err_v = np.zeros_like(p)
    abs_m = np.zeros_like(p)       # recursion on |terms| bounding intermediate sizes
    out, bounds = [], []
    for t in range(1, T + 1):
        w1 = np.array([omb1 * b1 ** (t - k) for k in range(1, t + 1)])
        w2 = np.array([omb2 * b2 ** (t - k) for k in range(1, t + 1)])
        m = w1 @ G[:t]
        v = w2 @ (G[:t] ** 2)
        bc1 = f64(1.0 - b1 ** t)
        bc2 = f64(1.0 - b2 ** t)
        mh, vh = m / bc1, v / bc2
        den = np.sqrt(vh) + eps
        upd = lr * mh / den
        # fp32 recursion errors: two products and a sum per step, each <= u
        err_m = b1 * err_m + 3 * U * (b1 * abs_m + omb1 * np.abs(G[t - 1]))
        abs_m = b1 * abs_m + omb1 * np.abs(G[t - 1])
        err_v = b2 * err_v + 4 * U * v
        # relative error of the denominator and absolute error of the update
        rel_den = 0.5 * (err_v / np.maximum(v, 1e-300) + 2 * U) + 3 * U
        err_upd = lr * (err_m / bc1 + 2 * U * abs_m / bc1) / den \
            + np.abs(upd) * (rel_den + 3 * U)
        p = p - upd
        err_p = err_p + err_upd + U * np.abs(p)
        out.append(p.copy())
        bounds.append(err_p.copy())
    return out, bounds


@pytest.mark.parametrize("seed,hp", [(0, (LR, B1, B2, EPS)), (1, (3e-4, 0.8, 0.95, 1e-6)),
                                     (2, (1e-2, 0.9, 0.999, 1e-8))])
def test_multi_step_against_unrolled_float64(seed, hp):
    lr, b1, b2, eps = hp
    n, T = 2000, 12
    rng = np.random.default_rng(seed)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gs = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(T)]
    ref, bounds = unrolled_reference(p0, gs, lr, b1, b2, eps)
    p, m, v, w = fresh(n)
    p[:] = p0
    for t in range(1, T + 1):
        oracle.adam_elems(p, m, v, w, gs[t - 1], lr, b1, b2, eps, t)
        err = np.abs(p.astype(np.float64) - ref[t - 1])
        assert np.all(err <= 4 * bounds[t - 1] + 1e-12), (t, (err / bounds[t - 1]).max())
        assert np.array_equal(w, torch_bf16_bits(p))


def test_step_size_bound():
    """Kingma & Ba, section 2.1: with (1-b1) > sqrt(1-b2) the effective step
    is bounded by lr (1-b1)/sqrt(1-b2)."""
    n, T = 5000, 20
    rng = np.random.default_rng(9)
    p, m, v, w = fresh(n)
    bound = LR * (1 - B1) / np.sqrt(1 - B2) * (1 + 1e-5)
    for t in range(1, T + 1):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 0, n)).astype(np.float32)
        before = p.astype(np.float64).copy()
        oracle.adam_elems(p, m, v, w, g, LR, B1, B2, EPS, t)
        assert np.abs(p - before).max() <= bound


def test_pads_untouched_and_only_owned_slice_updated():
    numels, nd = [10, 7, 3], 4
    L = oracle.Layout(numels, nd)
    for j in range(nd):
        sentinel = np.float32(7.0)
        p = np.full(L.S, sentinel, np.float32)
        m = np.full(L.S, sentinel, np.float32)
        v = np.full(L.S, sentinel, np.float32)
        w = np.full(L.S, 0x40e0, np.uint16)
        g = np.ones(L.S, np.float32)
        oracle.adam(numels, nd, j, p, m, v, w, g, LR, B1, B2, EPS, 1)
        t, i = L.locate(np.arange(L.S))
        pad = (j * L.shard_len[t] + i) >= L.numel[t]
        assert np.all(p[pad] == sentinel) and np.all(w[pad] == 0x40e0)
        assert np.all(m[pad] == sentinel) and np.all(v[pad] == sentinel)
        assert np.all(p[~pad] != sentinel)


def test_bf16_cast_matches_torch():
    """Round to nearest even, checked against torch's fp32 -> bf16 cast over
    random values of every magnitude plus ties, signed zeros, subnormals,
    the largest finite values and infinities."""
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x807fffff, 0x00008000,
                        0x00018000, 0x3f808000, 0x3f818000, 0x3f80ffff, 0x7f7fffff,
                        0xff7fffff, 0x7f7f8000, 0x7f7f7fff, 0x7f800000, 0xff800000,
                        0x3f7fffff, 0x33800000, 0x00400000], np.uint32)
    bits = np.concatenate([bits, special])
    x = bits.view(np.float32)
    finite = ~np.isnan(x)
    got = oracle.bf16_rne(x)
    ref = torch_bf16_bits(x)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(np.isnan(oracle.bf16_to_f32(got[~finite])))


def test_bf16_cast_nan_rule():
    """NaN inputs: the result is a quiet NaN of the same sign whose payload is
    the input payload's leading bits -- the IEEE 754 recommendation for
    narrowing a NaN (keep the payload as far as it fits, set the quiet bit).
    Checked as two properties over every bf16 NaN pattern: a quiet bf16 NaN
    widened to fp32 (bits << 16) and cast back is unchanged, and a signalling
    one comes back quieted with sign and payload kept; then fp32 NaNs with low
    payload bits set, which the narrowing drops."""
    hi = np.arange(1 << 16, dtype=np.uint32)
    nan16 = hi[((hi & 0x7f80) == 0x7f80) & ((hi & 0x007f) != 0)]
    quiet = nan16[(nan16 & 0x0040) != 0]
    signalling = nan16[(nan16 & 0x0040) == 0]
    back = oracle.bf16_rne((quiet << 16).astype(np.uint32).view(np.float32))
    assert np.array_equal(back.astype(np.uint32), quiet)
    back = oracle.bf16_rne((signalling << 16).astype(np.uint32).view(np.float32))
    assert np.array_equal(back.astype(np.uint32), signalling | 0x0040)
    low = np.array([0x7f800001, 0xff800001, 0x7fc00001, 0xffffffff, 0x7fbfffff, 0x7fa0ffff],
                   np.uint32)
    got = oracle.bf16_rne(low.view(np.float32)).astype(np.uint32)
    assert np.array_equal(got, (low >> 16) | 0x0040)
