"""ctypes binding of libzsp (include/zsp.h), one function per C entry point.

Argument marshalling only: torch tensors become raw device pointers, torch's
current stream becomes the hipStream_t, Python lists become C arrays. Every
step of the path runs in libzsp's HIP kernels. There is no fallback: if
libzsp.so is missing, importing this module raises.
"""
import ctypes
import os
import weakref

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzsp.so")

OK, EINVAL, ERANGE, ENOMEM, EHIP, ESTATE, EIO = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
GRADS_FULL, GRADS_SHARD = 0, 1
SRC_WORK, SRC_MASTER, SRC_ACC = 0, 1, 2
ALL_RANKS = -1
MAX_RANKS = 256

_STATUS_NAMES = {EINVAL: "ZSP_EINVAL", ERANGE: "ZSP_ERANGE", ENOMEM: "ZSP_ENOMEM",
                 EHIP: "ZSP_EHIP", ESTATE: "ZSP_ESTATE", EIO: "ZSP_EIO"}


class ZspError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    sigs = {
        "zsp_partition": (i32, [i64p, i32, i32, ctypes.POINTER(vp)]),
        "zsp_destroy": (None, [vp]),
        "zsp_plan_info": (i32, [vp, i64p, i64p, i64p]),
        "zsp_plan_tensor": (i32, [vp, i32, i64p, i64p, i64p, i64p, i64p]),
        "zsp_bind_state": (i32, [vp, i32, vp, vp, vp, vp, vp]),
        "zsp_load_params": (i32, [vp, vp, i32, vp]),
        "zsp_reduce_shard": (i32, [vp, i32, vpp, i32, i32, i32, vp]),
        "zsp_adam_step": (i32, [vp, i32, f32, f32, f32, f32, i64, vp]),
        "zsp_reduce_adam_step": (i32, [vp, i32, vpp, i32, i32, i32, f32, f32, f32, f32, i64,
                                       vp]),
        "zsp_reduce_shard_params": (i32, [vp, i32, i32, i32, vpp, i32, i32, i32, vp]),
        "zsp_adam_step_params": (i32, [vp, i32, i32, i32, f32, f32, f32, f32, i64, vp]),
        "zsp_reduce_adam_step_params": (i32, [vp, i32, i32, i32, vpp, i32, i32, i32, f32, f32,
                                              f32, f32, i64, vp]),
        "zsp_gather": (i32, [vp, i32, i32, vp, vp]),
        "zsp_gather_range": (i32, [vp, i32, i32, i32, vp, vp]),
        "zsp_gather_many": (i32, [vp, i32p, i32, i32, vpp, vp]),
        "zsp_gather_many_noalloc": (i32, [vp, i32p, i32, i32, vpp, vp]),
        "zsp_gather_list_create": (i32, [vp, i32p, i32, i32, vpp, vp, ctypes.POINTER(vp)]),
        "zsp_gather_list_run": (i32, [vp, vp]),
        "zsp_gather_list_destroy": (None, [vp]),
        "zsp_checkpoint_write_host": (i32, [vp, i32, ctypes.c_char_p, i64, vp, vp, vp, vp]),
        "zsp_checkpoint_read_host": (i32, [vp, i32, ctypes.c_char_p, i64p, vp, vp, vp, vp]),
        "zsp_checkpoint_save": (i32, [vp, i32, ctypes.c_char_p, i64, vp]),
        "zsp_checkpoint_load": (i32, [vp, i32, ctypes.c_char_p, i64p, vp]),
        "zsp_sched_create": (i32, [vp, i32, i32p, i32p, i32, i32p, i32, i32, i64p,
                                   ctypes.POINTER(vp)]),
        "zsp_sched_bind": (i32, [vp, vp, i64, vp]),
        "zsp_sched_acquire": (i32, [vp, i32, vp, ctypes.POINTER(vp)]),
        "zsp_sched_release": (i32, [vp, i32, vp]),
        "zsp_sched_reset": (i32, [vp]),
        "zsp_sched_set_engine": (i32, [vp, i32]),
        "zsp_sched_info": (i32, [vp, i32p, i32p, i64p]),
        "zsp_sched_destroy": (None, [vp]),
        "zsp_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def last_error():
    return lib.zsp_last_error().decode(errors="replace")


def _check(status):
    if status != OK:
        raise ZspError(status, last_error())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, dtype, what):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _grad_array(grads, n_d, min_elems=0):
    if len(grads) != n_d:
        raise ValueError(f"need {n_d} gradient buffers, got {len(grads)}")
    dt = grads[0].dtype
    for i, g in enumerate(grads):
        if isinstance(g, torch.Tensor) and g.numel() < min_elems:
            raise ValueError(f"grads[{i}] holds {g.numel()} elements; this layout reads "
                             f"{min_elems}")
    ptrs = [_ptr(g, dt, f"grads[{i}]").value for i, g in enumerate(grads)]
    return (ctypes.c_void_p * n_d)(*ptrs), _dtype_code(grads[0])


def _need(t, n, what):
    if t is not None and t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements; {n} are needed")


_LAYOUTS = {"full": GRADS_FULL, "shard": GRADS_SHARD, GRADS_FULL: GRADS_FULL,
            GRADS_SHARD: GRADS_SHARD}
_SOURCES = {"work": SRC_WORK, "master": SRC_MASTER, "acc": SRC_ACC, SRC_WORK: SRC_WORK,
            SRC_MASTER: SRC_MASTER, SRC_ACC: SRC_ACC}


# ---- one function per C entry point ---------------------------------------

def zsp_partition(numel, n_d):
    arr = (ctypes.c_int64 * len(numel))(*[int(n) for n in numel])
    h = ctypes.c_void_p()
    _check(lib.zsp_partition(arr, len(numel), int(n_d), ctypes.byref(h)))
    return h


def zsp_destroy(h):
    lib.zsp_destroy(h)


def zsp_plan_info(h):
    out = [ctypes.c_int64() for _ in range(3)]
    _check(lib.zsp_plan_info(h, *[ctypes.byref(o) for o in out]))
    return dict(zip(("shard_elems", "total_padded", "model_state_bytes_per_rank"),
                    (o.value for o in out)))


def zsp_plan_tensor(h, t):
    out = [ctypes.c_int64() for _ in range(5)]
    _check(lib.zsp_plan_tensor(h, int(t), *[ctypes.byref(o) for o in out]))
    return dict(zip(("numel", "pad", "shard_len", "full_off", "shard_off"),
                    (o.value for o in out)))


def zsp_bind_state(h, rank, master, m, v, work, grad_acc=None):
    _check(lib.zsp_bind_state(
        h, int(rank), _ptr(master, torch.float32, "master"), _ptr(m, torch.float32, "m"),
        _ptr(v, torch.float32, "v"), _ptr(work, torch.bfloat16, "work"),
        _ptr(grad_acc, torch.float32, "grad_acc")))


def zsp_load_params(h, flat, stream=None):
    _check(lib.zsp_load_params(h, _ptr(flat, flat.dtype, "flat_params"), _dtype_code(flat),
                               _stream(stream)))


def zsp_reduce_shard(h, n_d, rank, grads, layout="full", accumulate=False, stream=None,
                     min_elems=0):
    arr, code = _grad_array(grads, n_d, min_elems)
    _check(lib.zsp_reduce_shard(h, int(rank), arr, code, _LAYOUTS[layout], int(bool(accumulate)),
                                _stream(stream)))


def zsp_adam_step(h, rank, lr, beta1, beta2, eps, step, stream=None):
    _check(lib.zsp_adam_step(h, int(rank), float(lr), float(beta1), float(beta2), float(eps),
                             int(step), _stream(stream)))


def zsp_reduce_adam_step(h, n_d, rank, grads, lr, beta1, beta2, eps, step, layout="full",
                         use_acc=False, stream=None, min_elems=0):
    arr, code = _grad_array(grads, n_d, min_elems)
    _check(lib.zsp_reduce_adam_step(h, int(rank), arr, code, _LAYOUTS[layout],
                                    int(bool(use_acc)), float(lr), float(beta1), float(beta2),
                                    float(eps), int(step), _stream(stream)))


def zsp_reduce_shard_params(h, n_d, rank, first, n, grads, layout="full", accumulate=False,
                            stream=None, min_elems=0):
    arr, code = _grad_array(grads, n_d, min_elems)
    _check(lib.zsp_reduce_shard_params(h, int(rank), int(first), int(n), arr, code,
                                       _LAYOUTS[layout], int(bool(accumulate)), _stream(stream)))


def zsp_adam_step_params(h, rank, first, n, lr, beta1, beta2, eps, step, stream=None):
    _check(lib.zsp_adam_step_params(h, int(rank), int(first), int(n), float(lr), float(beta1),
                                    float(beta2), float(eps), int(step), _stream(stream)))


def zsp_reduce_adam_step_params(h, n_d, rank, first, n, grads, lr, beta1, beta2, eps, step,
                                layout="full", use_acc=False, stream=None, min_elems=0):
    arr, code = _grad_array(grads, n_d, min_elems)
    _check(lib.zsp_reduce_adam_step_params(h, int(rank), int(first), int(n), arr, code,
                                           _LAYOUTS[layout], int(bool(use_acc)), float(lr),
                                           float(beta1), float(beta2), float(eps), int(step),
                                           _stream(stream)))


def zsp_gather(h, param_id, out, source="work", stream=None):
    src = _SOURCES[source]
    dt = torch.bfloat16 if src == SRC_WORK else torch.float32
    _check(lib.zsp_gather(h, int(param_id), src, _ptr(out, dt, "out"), _stream(stream)))


def zsp_gather_range(h, first, n, out, source="work", stream=None):
    src = _SOURCES[source]
    dt = torch.bfloat16 if src == SRC_WORK else torch.float32
    _check(lib.zsp_gather_range(h, int(first), int(n), src, _ptr(out, dt, "out"),
                                _stream(stream)))


def _list_arrays(ids, outs, dt):
    if len(ids) != len(outs):
        raise ValueError(f"{len(ids)} ids but {len(outs)} outputs")
    n = len(ids)
    ids_c = (ctypes.c_int32 * max(n, 1))(*[int(i) for i in ids])
    ptrs = [None if o is None else _ptr(o, dt, f"outs[{i}]").value for i, o in enumerate(outs)]
    return ids_c, (ctypes.c_void_p * max(n, 1))(*ptrs), n


def zsp_gather_many(h, ids, outs, source="work", stream=None):
    src = _SOURCES[source]
    dt = torch.bfloat16 if src == SRC_WORK else torch.float32
    ids_c, outs_c, n = _list_arrays(ids, outs, dt)
    _check(lib.zsp_gather_many(h, ids_c, n, src, outs_c, _stream(stream)))


def zsp_gather_many_noalloc(h, ids, outs, source="work", stream=None):
    src = _SOURCES[source]
    dt = torch.bfloat16 if src == SRC_WORK else torch.float32
    ids_c, outs_c, n = _list_arrays(ids, outs, dt)
    _check(lib.zsp_gather_many_noalloc(h, ids_c, n, src, outs_c, _stream(stream)))


def zsp_gather_list_create(h, ids, outs, source="work", stream=None):
    """A prepared list gather (zsp_gather_list_create); returns its handle."""
    src = _SOURCES[source]
    dt = torch.bfloat16 if src == SRC_WORK else torch.float32
    ids_c, outs_c, n = _list_arrays(ids, outs, dt)
    out = ctypes.c_void_p()
    _check(lib.zsp_gather_list_create(h, ids_c, n, src, outs_c, _stream(stream),
                                      ctypes.byref(out)))
    return out


def zsp_gather_list_run(gl, stream=None):
    _check(lib.zsp_gather_list_run(gl, _stream(stream)))


def zsp_gather_list_destroy(gl):
    lib.zsp_gather_list_destroy(gl)


class GatherList:
    """A list gather prepared once (zsp_gather_list_create) for a caller that
    gathers the same bucket into the same outputs again and again (a
    module's parameters each step): each run is one launch. Keeps the plan
    and the outputs alive; frees the native list when collected or closed."""

    def __init__(self, plan, ids, outs, source="work", stream=None):
        self.plan = plan
        self.ids, self.outs = list(ids), list(outs)
        self._gl = zsp_gather_list_create(plan._h, self.ids, self.outs, source, stream)
        plan._lists.add(self)

    def run(self, stream=None):
        if self._gl is None:
            raise ValueError("gather list is closed")
        zsp_gather_list_run(self._gl, stream)

    def close(self):
        """Frees the native list; runs already enqueued must have finished."""
        if getattr(self, "_gl", None) is not None:
            zsp_gather_list_destroy(self._gl)
            self._gl = None

    def __del__(self):
        self.close()


def _host_arrays(S, master, m, v, work, writable):
    import numpy as np
    out = []
    for a, dt, name in ((master, np.float32, "master"), (m, np.float32, "m"),
                        (v, np.float32, "v"), (work, np.uint16, "work")):
        if not isinstance(a, np.ndarray) or a.dtype != dt or not a.flags.c_contiguous:
            raise TypeError(f"{name} must be a contiguous numpy {dt.__name__} array")
        if a.size < S or (writable and not a.flags.writeable):
            raise ValueError(f"{name} must hold {S} elements" + (" and be writable" if writable else ""))
        out.append(ctypes.c_void_p(a.ctypes.data))
    return out


def zsp_checkpoint_write_host(h, rank, directory, step, master, m, v, work):
    """Write one rank's shard set from host numpy arrays (float32 x3, uint16 bf16 bits)."""
    S = zsp_plan_info(h)["shard_elems"]
    _check(lib.zsp_checkpoint_write_host(h, int(rank), str(directory).encode(), int(step),
                                         *_host_arrays(S, master, m, v, work, False)))


def zsp_checkpoint_read_host(h, rank, directory, master, m, v, work):
    """Read (resharding if needed) one rank's shard set into host numpy arrays; returns step."""
    S = zsp_plan_info(h)["shard_elems"]
    step = ctypes.c_int64()
    _check(lib.zsp_checkpoint_read_host(h, int(rank), str(directory).encode(), ctypes.byref(step),
                                        *_host_arrays(S, master, m, v, work, True)))
    return step.value


def zsp_checkpoint_save(h, rank, directory, step, stream=None):
    _check(lib.zsp_checkpoint_save(h, int(rank), str(directory).encode(), int(step),
                                   _stream(stream)))


def zsp_checkpoint_load(h, rank, directory, stream=None):
    step = ctypes.c_int64()
    _check(lib.zsp_checkpoint_load(h, int(rank), str(directory).encode(), ctypes.byref(step),
                                   _stream(stream)))
    return step.value


# ---- per-layer gather schedule -----------------------------------------------

def _i32_array(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_int32 * max(len(xs), 1))(*xs), len(xs)


def zsp_sched_create(h, groups, order, depth, source="work"):
    """groups: [(first_param, n_params), ...]; order: group index per position.
    Returns (handle, arena_bytes)."""
    first, n_groups = _i32_array(g[0] for g in groups)
    count, _ = _i32_array(g[1] for g in groups)
    order_c, n_steps = _i32_array(order)
    src = SRC_WORK if source == "work" else SRC_MASTER
    nbytes = ctypes.c_int64()
    out = ctypes.c_void_p()
    _check(lib.zsp_sched_create(h, n_groups, first, count, n_steps, order_c, int(depth), src,
                                ctypes.byref(nbytes), ctypes.byref(out)))
    return out, nbytes.value


def zsp_sched_bind(s, arena, gather_stream):
    if not isinstance(arena, torch.Tensor) or not arena.is_cuda or not arena.is_contiguous():
        raise TypeError("arena must be a contiguous torch tensor on the GPU")
    gs = None if gather_stream is None else _stream(gather_stream)
    _check(lib.zsp_sched_bind(s, ctypes.c_void_p(arena.data_ptr()),
                              arena.numel() * arena.element_size(), gs))


def zsp_sched_acquire(s, position, stream=None):
    """Returns the device address of the position's gathered group."""
    out = ctypes.c_void_p()
    _check(lib.zsp_sched_acquire(s, int(position), _stream(stream), ctypes.byref(out)))
    return out.value


def zsp_sched_release(s, position, stream=None):
    _check(lib.zsp_sched_release(s, int(position), _stream(stream)))


def zsp_sched_reset(s):
    _check(lib.zsp_sched_reset(s))


ENGINE_KERNEL, ENGINE_COPY = 0, 1
_ENGINES = {"kernel": ENGINE_KERNEL, "copy": ENGINE_COPY, ENGINE_KERNEL: ENGINE_KERNEL,
            ENGINE_COPY: ENGINE_COPY}


def zsp_sched_set_engine(s, engine):
    _check(lib.zsp_sched_set_engine(s, _ENGINES[engine]))


def zsp_sched_info(s):
    d, n, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib.zsp_sched_info(s, ctypes.byref(d), ctypes.byref(n), ctypes.byref(b)))
    return {"depth": d.value, "slots": n.value, "slot_bytes": b.value}


def zsp_sched_destroy(s):
    lib.zsp_sched_destroy(s)


class Schedule:
    """Owns a zsp_sched handle over a Plan. acquire() returns the
    position's gathered parameters as tensor views of the arena, one per
    parameter of its group (unpadded, flattened)."""

    def __init__(self, plan, groups, order, depth, source="work"):
        self.plan = plan
        self.groups = [(int(f), int(c)) for f, c in groups]
        self.order = [int(g) for g in order]
        self.dtype = torch.bfloat16 if source == "work" else torch.float32
        if plan._h is None:
            raise ZspError(ESTATE, "the plan is destroyed")
        self._h, self.arena_bytes = zsp_sched_create(plan._h, self.groups, self.order, depth,
                                                     source)
        self.info = zsp_sched_info(self._h)
        self.arena = None
        plan._schedules.add(self)

    def _live(self):
        if self._h is None:
            raise ZspError(ESTATE, "the schedule is destroyed (or its plan is)")
        return self._h

    def set_engine(self, engine):
        """'kernel' or 'copy' (the DMA copy engines); bind again after."""
        zsp_sched_set_engine(self._live(), engine)
        self.arena = None

    def bind(self, arena, gather_stream):
        zsp_sched_bind(self._live(), arena, gather_stream)
        self.arena = arena

    def acquire(self, position, stream=None):
        addr = zsp_sched_acquire(self._live(), position, stream)
        off = addr - self.arena.data_ptr()
        first, count = self.groups[self.order[position]]
        esz = torch.finfo(self.dtype).bits // 8
        flat = self.arena.view(torch.uint8)[off:off + esz * sum(
            self.plan.numel[first:first + count])].view(self.dtype)
        views, k = [], 0
        for t in range(first, first + count):
            views.append(flat[k:k + self.plan.numel[t]])
            k += self.plan.numel[t]
        return views

    def release(self, position, stream=None):
        zsp_sched_release(self._live(), position, stream)

    def reset(self):
        zsp_sched_reset(self._live())

    def destroy(self):
        if self._h:
            zsp_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


# ---- a plan object over the same calls -------------------------------------

class Plan:
    """Owns a zsp_plan handle; methods map one-to-one onto the C calls."""

    def __init__(self, numel, n_d):
        self.numel = [int(n) for n in numel]
        self.n_d = int(n_d)
        self._h = zsp_partition(self.numel, self.n_d)
        info = zsp_plan_info(self._h)
        self.S = info["shard_elems"]
        self.total_padded = info["total_padded"]
        self.total_numel = sum(self.numel)
        self.flat_off = [0]
        for n in self.numel:
            self.flat_off.append(self.flat_off[-1] + n)
        self.model_state_bytes_per_rank = info["model_state_bytes_per_rank"]
        self._bound = None
        self._bound_rank = None
        self._schedules = weakref.WeakSet()   # destroyed before the plan
        self._lists = weakref.WeakSet()       # prepared gather lists, likewise

    @property
    def handle(self):
        return self._h

    def destroy(self):
        for sched in list(self._schedules):
            sched.destroy()
        for gl in list(self._lists):
            gl.close()
        if self._h is not None and self._h.value:
            zsp_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def info(self):
        return zsp_plan_info(self._h)

    def tensor(self, t):
        """Parameter t's layout (zsp_plan_tensor), with flat_off: its offset
        in the unpadded concatenation."""
        d = zsp_plan_tensor(self._h, t)
        d["flat_off"] = self.flat_off[t]
        return d

    # The C calls take raw pointers and cannot see buffer sizes; these methods
    # check every tensor against the plan before anything is launched.

    def _state_elems(self):
        if self._bound_rank is None:
            return 0
        return self.S * (self.n_d if self._bound_rank == ALL_RANKS else 1)

    def _grad_elems(self, layout):
        return self.total_padded if _LAYOUTS[layout] == GRADS_FULL else self._state_elems()

    def bind_state(self, rank, master, m, v, work, grad_acc=None):
        n = self.S * (self.n_d if rank == ALL_RANKS else 1)
        for t, name in ((master, "master"), (m, "m"), (v, "v"), (work, "work"),
                        (grad_acc, "grad_acc")):
            _need(t, n, name)
        zsp_bind_state(self._h, rank, master, m, v, work, grad_acc)
        # keep the tensors alive for as long as they are bound
        self._bound = (master, m, v, work, grad_acc)
        self._bound_rank = rank

    def load_params(self, flat, stream=None):
        _need(flat, self.total_numel, "flat_params")
        zsp_load_params(self._h, flat, stream)

    def reduce_shard(self, rank, grads, layout="full", accumulate=False, stream=None):
        zsp_reduce_shard(self._h, self.n_d, rank, grads, layout, accumulate, stream,
                         self._grad_elems(layout))

    def adam_step(self, rank, lr, beta1, beta2, eps, step, stream=None):
        zsp_adam_step(self._h, rank, lr, beta1, beta2, eps, step, stream)

    def reduce_adam_step(self, rank, grads, lr, beta1, beta2, eps, step, layout="full",
                         use_acc=False, stream=None):
        zsp_reduce_adam_step(self._h, self.n_d, rank, grads, lr, beta1, beta2, eps, step,
                             layout, use_acc, stream, self._grad_elems(layout))

    def reduce_shard_params(self, rank, first, n, grads, layout="full", accumulate=False,
                            stream=None):
        zsp_reduce_shard_params(self._h, self.n_d, rank, first, n, grads, layout, accumulate,
                                stream, self._grad_elems(layout))

    def adam_step_params(self, rank, first, n, lr, beta1, beta2, eps, step, stream=None):
        zsp_adam_step_params(self._h, rank, first, n, lr, beta1, beta2, eps, step, stream)

    def reduce_adam_step_params(self, rank, first, n, grads, lr, beta1, beta2, eps, step,
                                layout="full", use_acc=False, stream=None):
        zsp_reduce_adam_step_params(self._h, self.n_d, rank, first, n, grads, lr, beta1, beta2,
                                    eps, step, layout, use_acc, stream, self._grad_elems(layout))

    def gather(self, param_id, out, source="work", stream=None):
        if 0 <= param_id < len(self.numel):
            _need(out, self.numel[param_id], "out")
        zsp_gather(self._h, param_id, out, source, stream)

    def gather_range(self, first, n, out, source="work", stream=None):
        if 0 <= first and n >= 1 and first + n <= len(self.numel):
            _need(out, sum(self.numel[first:first + n]), "out")
        zsp_gather_range(self._h, first, n, out, source, stream)

    def gather_many(self, ids, outs, source="work", stream=None):
        """Parameter ids[i] into outs[i] (a tensor of at least its numel
        elements; None for an empty parameter), all in one call."""
        for i, (t, o) in enumerate(zip(ids, outs)):
            if 0 <= t < len(self.numel):
                _need(o, self.numel[t], f"outs[{i}]")
        zsp_gather_many(self._h, ids, outs, source, stream)

    def gather_many_noalloc(self, ids, outs, source="work", stream=None):
        """gather_many staged through the library's fixed device array:
        allocates nothing."""
        for i, (t, o) in enumerate(zip(ids, outs)):
            if 0 <= t < len(self.numel):
                _need(o, self.numel[t], f"outs[{i}]")
        zsp_gather_many_noalloc(self._h, ids, outs, source, stream)

    def gather_list(self, ids, outs, source="work"):
        """A prepared GatherList for this plan's parameters (sizes checked
        and records built once); run it with gather_prepared."""
        for i, (t, o) in enumerate(zip(ids, outs)):
            if 0 <= t < len(self.numel):
                _need(o, self.numel[t], f"outs[{i}]")
        return GatherList(self, ids, outs, source)

    def gather_prepared(self, glist, stream=None):
        glist.run(stream)

    def checkpoint_save(self, rank, directory, step, stream=None):
        zsp_checkpoint_save(self._h, rank, directory, step, stream)

    def checkpoint_load(self, rank, directory, stream=None):
        return zsp_checkpoint_load(self._h, rank, directory, stream)

    def checkpoint_write_host(self, rank, directory, step, master, m, v, work):
        zsp_checkpoint_write_host(self._h, rank, directory, step, master, m, v, work)

    def checkpoint_read_host(self, rank, directory, master, m, v, work):
        return zsp_checkpoint_read_host(self._h, rank, directory, master, m, v, work)


def partition(numel, n_d):
    """partition(param list, N_d) -> Plan."""
    return Plan(numel, n_d)
