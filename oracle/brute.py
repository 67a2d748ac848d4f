"""A second CPU implementation of the per-rank step, for tiny inputs only.

TEST INFRASTRUCTURE ONLY: only ``tests/`` import it. It shares no code with
``oracle.c`` and is written differently on purpose, so that agreeing with it
bit for bit checks the C oracle's *implementation* (a wrong slice or offset,
a slip in the order of operations, an fp32 operation contracted into an FMA
or carried out in higher precision by the compiler), while the mathematics
itself is pinned by the closed forms and bounds in ``tests/test_oracle_*``:

* Layout ("The ZeRO-3 Diagram Most People Remember Is Wrong", section 2):
  each parameter is materialised as a Python list of its element indices,
  padded with ``None`` up to a multiple of the rank count and cut into that
  many equal slices; the tables are read off those lists.
* Reduce ("ZeRO Stages...", "Stage 2 also partitions gradients"): the ranks'
  values added one numpy float32 scalar at a time, rank 0 first.
* Adam (Kingma & Ba, "Adam: A Method for Stochastic Optimization",
  Algorithm 1): one numpy float32 scalar operation per step of the
  algorithm, each rounded to nearest-even; the bias corrections 1 - beta^t
  computed in double and rounded once to fp32.
* bf16 narrowing: by value, in exact rational arithmetic (the nearest bf16
  number, ties to the even significand), where the C oracle rounds on the
  dropped bits. NaN has no value; it is quieted keeping its sign and the
  leading bits of its payload (IEEE 754's recommendation for narrowing).
"""
import math
from fractions import Fraction

import numpy as np

F32 = np.float32


# ---- layout -----------------------------------------------------------------

def layout(numel, nd):
    """Per-parameter tables from padded, sliced index lists."""
    pads, shard_len, full_off, shard_off, flat_off = [], [], [0], [0], [0]
    for n in numel:
        elems = list(range(n))
        while len(elems) % nd:
            elems.append(None)
        slices = [elems[r * (len(elems) // nd):(r + 1) * (len(elems) // nd)] for r in range(nd)]
        assert sum(len(s) for s in slices) == len(elems)
        pads.append(len(elems) - n)
        shard_len.append(len(slices[0]))
        full_off.append(full_off[-1] + len(elems))
        shard_off.append(shard_off[-1] + len(slices[0]))
        flat_off.append(flat_off[-1] + n)
    return {"pad": pads, "shard_len": shard_len, "full_off": full_off,
            "shard_off": shard_off, "flat_off": flat_off, "S": shard_off[-1]}


def owners(numel, nd):
    """For rank j: the list, over its S shard positions, of (t, i) -- parameter
    t's element i -- or None for a pad position."""
    out = [[] for _ in range(nd)]
    for t, n in enumerate(numel):
        elems = list(range(n))
        while len(elems) % nd:
            elems.append(None)
        s = len(elems) // nd
        for r in range(nd):
            out[r].extend(None if i is None else (t, i) for i in elems[r * s:(r + 1) * s])
    return out


# ---- bf16 -------------------------------------------------------------------

def f32_bits(x):
    return int(np.array([x], F32).view(np.uint32)[0])


def f32_of_bits(u):
    return np.array([u], np.uint32).view(F32)[0]


def bf16_widen(h):
    """The fp32 value of bf16 bits h (bf16 is fp32 with 16 fewer significand
    bits, so this is exact)."""
    return f32_of_bits(int(h) << 16)


def bf16_widen_array(bits):
    """bf16_widen of every element of a sequence of bf16 bit patterns."""
    return [bf16_widen(h) for h in bits]


def bf16(x):
    """bf16 bits of the fp32 value x, rounded to nearest, ties to even."""
    x = F32(x)
    u = f32_bits(x)
    sign = (u >> 16) & 0x8000
    if math.isnan(float(x)):
        return (u >> 16) | 0x0040
    if math.isinf(float(x)) or x == 0:
        return u >> 16
    a = Fraction(abs(float(x)))
    _, e = math.frexp(float(a))          # a = m * 2^e with 0.5 <= m < 1
    e -= 1                               # a in [2^e, 2^(e+1))
    quantum = Fraction(2) ** (max(e, -126) - 7)   # 8 significant bits; subnormal step 2^-133
    q, rem = divmod(a, quantum)
    q = int(q)
    if rem > quantum / 2 or (rem == quantum / 2 and q % 2 == 1):
        q += 1
    value = q * quantum
    if value >= Fraction(2) ** 128:
        return sign | 0x7f80
    return sign | (f32_bits(F32(float(value))) >> 16)


# ---- the step ----------------------------------------------------------------

def reduce_elem(values):
    """Rank-order fp32 sum of one element's N_d values."""
    acc = F32(values[0])
    for x in values[1:]:
        acc = F32(acc + F32(x))
    return acc


def adam_elem(p, m, v, g, lr, b1, b2, eps, t):
    """One element of one Adam step; returns the new (p, m, v)."""
    lr, b1, b2, eps, g = F32(lr), F32(b1), F32(b2), F32(eps), F32(g)
    one = F32(1.0)
    bc1 = F32(1.0 - float(b1) ** t)
    bc2 = F32(1.0 - float(b2) ** t)
    m_t = F32(b1 * F32(m)) + F32((one - b1) * g)
    v_t = F32(b2 * F32(v)) + F32((one - b2) * F32(g * g))
    m_hat = F32(m_t / bc1)
    v_hat = F32(v_t / bc2)
    den = F32(np.sqrt(v_hat) + eps)
    p_t = F32(F32(p) - F32(F32(lr * m_hat) / den))
    return p_t, F32(m_t), F32(v_t)


class Model:
    """Every rank's state for a tiny parameter list, held as Python lists."""

    def __init__(self, numel, nd, flat):
        self.numel, self.nd = list(numel), nd
        self.L = layout(numel, nd)
        self.own = owners(numel, nd)
        f = self.L["flat_off"]
        self.master, self.m, self.v, self.work = [], [], [], []
        for j in range(nd):
            vals = [F32(0.0) if o is None else F32(flat[f[o[0]] + o[1]]) for o in self.own[j]]
            self.master.append(vals)
            self.m.append([F32(0.0)] * len(vals))
            self.v.append([F32(0.0)] * len(vals))
            self.work.append([bf16(x) for x in vals])

    def grad_values(self, grads, j, k):
        """The N_d ranks' gradients (full padded layout, fp32 values) of rank
        j's shard position k."""
        t, i = self.own[j][k]
        idx = self.L["full_off"][t] + i      # element i of padded parameter t
        return [grads[r][idx] for r in range(self.nd)]

    def reduce(self, grads, j):
        """Rank j's reduced shard (None at pad positions)."""
        return [None if o is None else reduce_elem(self.grad_values(grads, j, k))
                for k, o in enumerate(self.own[j])]

    def step(self, grads, lr, b1, b2, eps, t, acc=None):
        """Reduce (added to acc[j] when given) and Adam on every rank."""
        for j in range(self.nd):
            red = self.reduce(grads, j)
            for k, g in enumerate(red):
                if g is None:
                    continue
                if acc is not None:
                    g = F32(acc[j][k] + g)
                p, m, v = adam_elem(self.master[j][k], self.m[j][k], self.v[j][k], g,
                                    lr, b1, b2, eps, t)
                self.master[j][k], self.m[j][k], self.v[j][k] = p, m, v
                self.work[j][k] = bf16(p)
