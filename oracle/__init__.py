"""CPU oracle for the per-rank hot path of ZeRO-3 intra-layer partitioning.

TEST INFRASTRUCTURE ONLY. The tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product package
never does. It wraps ``oracle/liboracle.so`` (plain C, see ``oracle.c``) with
numpy arrays: fp32 values are ``np.float32`` and bf16 values are their raw
bit patterns as ``np.uint16``.

Pages followed (by title and section):
  "The ZeRO-3 Diagram Most People Remember Is Wrong", sections 2 and 3
  "ZeRO Stage 3: Parameter Partitioning", on-demand fetch and eq. M_Stage3
  "ZeRO Stages: Sharding Optimizer State, Gradients, and Parameters"
The Adam update is the textbook one (Kingma & Ba, Algorithm 1); the pages
name Adam but do not print it.
"""
import ctypes
import os

import numpy as np

F32 = 0
BF16 = 1
GRADS_FULL = 0
GRADS_SHARD = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZSP_ORACLE_LIB lets the mutation test load a deliberately broken build.
_LIB_PATH = os.environ.get("ZSP_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_vp = ctypes.c_void_p


def lib():
    """Load liboracle.so, building it with gcc first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_pad.restype = ctypes.c_int64
        L.orc_pad.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.orc_layout.restype = ctypes.c_int
        L.orc_layout.argtypes = [ctypes.c_int32, _i64p, ctypes.c_int32,
                                 _i64p, _i64p, _i64p, _i64p, _i64p, _i64p]
        L.orc_model_state_bytes.restype = ctypes.c_int64
        L.orc_model_state_bytes.argtypes = [ctypes.c_int64]
        L.orc_stage_state_bytes.restype = ctypes.c_int64
        L.orc_stage_state_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int32]
        L.orc_stage_comm_elems.restype = ctypes.c_double
        L.orc_stage_comm_elems.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_bf16_rne_array.restype = None
        L.orc_bf16_rne_array.argtypes = [ctypes.c_int64, _f32p, _u16p]
        L.orc_partition.restype = ctypes.c_int
        L.orc_partition.argtypes = [ctypes.c_int32, _i64p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32,
                                    _f32p, _u16p, _f32p, _f32p]
        L.orc_reduce.restype = ctypes.c_int
        L.orc_reduce.argtypes = [ctypes.c_int32, _i64p, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.POINTER(_vp), ctypes.c_int32, ctypes.c_int32, _f32p]
        L.orc_reduce_values.restype = None
        L.orc_reduce_values.argtypes = [ctypes.c_int64, ctypes.c_int32, _vp,
                                        ctypes.c_int32, _f32p]
        L.orc_accumulate.restype = None
        L.orc_accumulate.argtypes = [ctypes.c_int64, _f32p, _f32p]
        L.orc_adam_scalars.restype = None
        L.orc_adam_scalars.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_int64, _f32p]
        L.orc_adam_elems.restype = None
        L.orc_adam_elems.argtypes = [ctypes.c_int64, _f32p, _f32p, _f32p, _u16p, _f32p,
                                     ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_float, ctypes.c_int64]
        L.orc_adam.restype = ctypes.c_int
        L.orc_adam.argtypes = [ctypes.c_int32, _i64p, ctypes.c_int32, ctypes.c_int32,
                               _f32p, _f32p, _f32p, _u16p, _f32p,
                               ctypes.c_float, ctypes.c_float, ctypes.c_float,
                               ctypes.c_float, ctypes.c_int64]
        L.orc_gather.restype = ctypes.c_int
        L.orc_gather.argtypes = [ctypes.c_int32, _i64p, ctypes.c_int32, ctypes.c_int32,
                                 _vp, ctypes.c_int32, _vp]
        _lib = L
    return _lib


def _p(a, ty):
    return a.ctypes.data_as(ty)


def _numel_arr(numel):
    a = np.ascontiguousarray(np.asarray(numel, dtype=np.int64).reshape(-1))
    return a


def _dtype_code(arr):
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {arr.dtype}")


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected its arguments")


def pad(numel, nd):
    return int(lib().orc_pad(int(numel), int(nd)))


class Layout:
    """Per-tensor layout tables computed by the oracle."""

    def __init__(self, numel, nd):
        n = _numel_arr(numel)
        T = n.size
        self.numel = n
        self.nd = int(nd)
        self.T = T
        self.pad = np.zeros(T, np.int64)
        self.shard_len = np.zeros(T, np.int64)
        self.full_off = np.zeros(T + 1, np.int64)
        self.shard_off = np.zeros(T + 1, np.int64)
        self.flat_off = np.zeros(T + 1, np.int64)
        S = np.zeros(1, np.int64)
        _check(lib().orc_layout(T, _p(n, _i64p), self.nd, _p(self.pad, _i64p),
                                _p(self.shard_len, _i64p), _p(self.full_off, _i64p),
                                _p(self.shard_off, _i64p), _p(self.flat_off, _i64p),
                                _p(S, _i64p)), "layout")
        self.S = int(S[0])
        self.padded = self.numel + self.pad

    @property
    def total_padded(self):
        return int(self.full_off[-1])

    @property
    def total_numel(self):
        return int(self.flat_off[-1])

    def locate(self, e):
        """Map shard positions e (array) to (tensor t, index i within its slice)."""
        e = np.asarray(e, dtype=np.int64)
        t = np.searchsorted(self.shard_off, e, side="right") - 1
        return t, e - self.shard_off[t]


def model_state_bytes(shard_elems):
    return int(lib().orc_model_state_bytes(int(shard_elems)))


def stage_state_bytes(stage, psi, shard_elems, grad_bytes=2):
    return int(lib().orc_stage_state_bytes(int(stage), int(psi), int(shard_elems),
                                           int(grad_bytes)))


def stage_comm_elems(stage, n, p):
    return float(lib().orc_stage_comm_elems(int(stage), int(n), int(p)))


def bf16_rne(x):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_rne_array(x.size, _p(x, _f32p), _p(out, _u16p))
    return out


def bf16_to_f32(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def partition(numel, nd, flat, rank_lo=0, rank_hi=None):
    """Copy-in of ranks [rank_lo, rank_hi): returns master, work(bf16 bits), m, v."""
    L = Layout(numel, nd)
    if rank_hi is None:
        rank_hi = L.nd
    flat = np.ascontiguousarray(flat)
    if flat.size < L.total_numel:
        raise ValueError("flat input shorter than the sum of numel")
    n = (rank_hi - rank_lo) * L.S
    master = np.empty(n, np.float32)
    work = np.empty(n, np.uint16)
    m = np.empty(n, np.float32)
    v = np.empty(n, np.float32)
    _check(lib().orc_partition(L.T, _p(L.numel, _i64p), L.nd, rank_lo, rank_hi,
                               flat.ctypes.data_as(_vp), _dtype_code(flat),
                               _p(master, _f32p), _p(work, _u16p), _p(m, _f32p),
                               _p(v, _f32p)), "partition")
    return master, work, m, v


def reduce(numel, nd, j, grads, layout=GRADS_FULL):
    """fp32 sum, in rank order, of the nd gradients into rank j's shard (S)."""
    L = Layout(numel, nd)
    if len(grads) != L.nd:
        raise ValueError("need one gradient buffer per rank")
    gs = [np.ascontiguousarray(g) for g in grads]
    need = L.total_padded if layout == GRADS_FULL else L.S
    code = _dtype_code(gs[0])
    for g in gs:
        if _dtype_code(g) != code or g.size < need:
            raise ValueError("gradient buffers must share a dtype and be large enough")
    ptrs = (_vp * L.nd)(*[g.ctypes.data for g in gs])
    out = np.empty(L.S, np.float32)
    _check(lib().orc_reduce(L.T, _p(L.numel, _i64p), L.nd, int(j), ptrs, code,
                            int(layout), _p(out, _f32p)), "reduce")
    return out


def reduce_values(vals):
    """vals: (n, nd) array of each rank's value for n elements -> fp32 sums (n,)."""
    vals = np.ascontiguousarray(vals)
    n, nd = vals.shape
    out = np.empty(n, np.float32)
    lib().orc_reduce_values(n, nd, vals.ctypes.data_as(_vp), _dtype_code(vals),
                            _p(out, _f32p))
    return out


def accumulate(acc, g):
    """acc <- acc + g (in place, fp32)."""
    assert acc.dtype == np.float32 and g.dtype == np.float32 and acc.flags.c_contiguous
    g = np.ascontiguousarray(g)
    lib().orc_accumulate(acc.size, _p(acc, _f32p), _p(g, _f32p))
    return acc


def adam_scalars(b1, b2, step):
    out = np.zeros(4, np.float32)
    lib().orc_adam_scalars(float(b1), float(b2), int(step), _p(out, _f32p))
    return out


def adam_elems(master, m, v, work, g, lr, b1, b2, eps, step):
    """Adam + bf16 refresh on plain element arrays (in place)."""
    for a, dt in ((master, np.float32), (m, np.float32), (v, np.float32),
                  (work, np.uint16)):
        assert a.dtype == dt and a.flags.c_contiguous
    g = np.ascontiguousarray(g, dtype=np.float32)
    lib().orc_adam_elems(master.size, _p(master, _f32p), _p(m, _f32p), _p(v, _f32p),
                         _p(work, _u16p), _p(g, _f32p), float(lr), float(b1),
                         float(b2), float(eps), int(step))


def adam(numel, nd, j, master, m, v, work, g, lr, b1, b2, eps, step):
    """Adam on rank j's shard (arrays of S elements, in place; pads untouched)."""
    L = Layout(numel, nd)
    for a, dt in ((master, np.float32), (m, np.float32), (v, np.float32),
                  (work, np.uint16)):
        assert a.dtype == dt and a.flags.c_contiguous and a.size >= L.S
    g = np.ascontiguousarray(g, dtype=np.float32)
    _check(lib().orc_adam(L.T, _p(L.numel, _i64p), L.nd, int(j), _p(master, _f32p),
                          _p(m, _f32p), _p(v, _f32p), _p(work, _u16p), _p(g, _f32p),
                          float(lr), float(b1), float(b2), float(eps), int(step)),
           "adam")


def gather(numel, nd, t, src):
    """Full unpadded tensor t from the nd*S shard array src (fp32 or bf16 bits)."""
    L = Layout(numel, nd)
    src = np.ascontiguousarray(src)
    if src.size < L.nd * L.S:
        raise ValueError("source must hold nd*S elements")
    out = np.empty(int(L.numel[t]), src.dtype)
    _check(lib().orc_gather(L.T, _p(L.numel, _i64p), L.nd, int(t),
                            src.ctypes.data_as(_vp), _dtype_code(src),
                            out.ctypes.data_as(_vp)), "gather")
    return out
