"""Benchmark of the ZeRO-3 per-rank hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  * the shard reduce of every virtual rank's gradient fused with the Adam
    step and the bf16 cast (one launch over all N_d ranks; with gradient
    accumulation, the earlier micro-batches' reduce launches first), then
  * the parameter gathers before forward and again before backward.
Inputs are seeded, synthetic and already resident in HBM when timing starts.

Metric: effective GB/s = algorithmic bytes / time, where algorithmic bytes
count what the method must move per real (non-pad) element:
  fused reduce+Adam+cast   N_d*g + 12 (read master, m, v) + 14 (write master,
                           m, v, bf16 work) [+ 4 reading the accumulator]
  reduce (accumulate)      N_d*g + 4 (write) [+ 4 read when accumulating]
  gather                   2*w (read shard, write full) per unpadded element
with g, w the gradient and parameter element sizes in bytes.

Prints one JSON line for --workload (default: the 8192x28672 MLP at N_d = 16
with 8 micro-batches, the largest workload; its step is seven reduce
launches, one fused reduce+accumulate+Adam+cast launch and the gathers):
the metric over the whole step, a roofline object for the kind of launch
that takes the most time per step (HIP-event time, peak, and HBM traffic
from stored PMC counters when they match the kernels' source), the CPU
oracle's figure on a bounded sample, and, under "workloads", the same
per-kernel figures for every other workload (--only skips them).

Other modes, each printing its own JSON line:
  --stage 1|2   the step in the ZeRO stage-1 or stage-2 schedule
  --split       reduce into the accumulator, then Adam (unfused update)
  --prefetch    forward + backward over a Llama-7B stack through the
                per-layer gather schedule; hidden fraction of gather time
  --checkpoint DIR   sharded checkpoint save / load / reshard-load timings
  --rocprof-summary DIR, --traffic-from F W   turn rocprofv3 output into the
                text and JSON summaries kept under profiles/
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
DEFAULT_WORKLOAD = "mlp8192x28672_accum_nd16"
METRIC = "effective GB/s (and % HBM peak) of shard reduce+Adam+cast step and param gather"
# Kinds of launch inside one step, in bench.py's event records.
STEP_KINDS = ("reduce_set", "reduce_acc", "fused", "adam", "gather_acc", "gather")
KERNEL_SOURCES = ["zero_sharded_mixed_pad_amd/csrc/zsp_kernels.hip",
                  "zero_sharded_mixed_pad_amd/csrc/zsp_internal.hpp"]


def _code_only(text):
    """C++ source without its comments and with runs of white space folded,
    so that editing a comment leaves the hash alone (string literals in the
    kernel sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of what determines the kernels' code: their source and header
    (comments aside) and the device compile flags (other library sources do
    not enter it)."""
    import importlib.util
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    spec = importlib.util.spec_from_file_location(
        "_zsp_build_flags", os.path.join(ROOT, "zero_sharded_mixed_pad_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    flags = [f for f in mod.FLAGS if not f.startswith("/")]
    h.update(repr((mod.ARCH, flags)).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", dest="all_workloads", action="store_false",
                    help="time only --workload (default: also every other workload, "
                         "reported under 'workloads')")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the oracle baseline sample")
    ap.add_argument("--flush", choices=["auto", "on", "off"], default="auto",
                    help="read a 1 GiB buffer before each step so a small working set is "
                         "not served from the 256 MB Infinity Cache (auto: fused step under "
                         "2 GB); gathers under 1 GB are also timed cold, after such a read")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain 2 GiB device copies (PMC byte-count calibration)")
    ap.add_argument("--rocprof-summary", metavar="DIR", default=None)
    ap.add_argument("--summary-out", default=None)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --calibrate-copy' into profiles/traffic_<workload>.json")
    ap.add_argument("--checkpoint", metavar="DIR", default=None,
                    help="instead of the step: time a sharded checkpoint save, load, and "
                         "load under half the rank count (reshard) of the workload's state "
                         "in a fresh directory under DIR, check the bits, print one JSON line")
    ap.add_argument("--stage", type=int, choices=[1, 2, 3], default=3,
                    help="ZeRO stage whose step schedule runs (3: the partitioned hot path)")
    ap.add_argument("--split", action="store_true",
                    help="unfused update: reduce into the accumulator, then Adam from it")
    ap.add_argument("--prefetch", action="store_true",
                    help="instead of the step: time forward+backward passes of a Llama-7B "
                         "decoder stack through the per-layer gather schedule at several "
                         "prefetch depths, with a matmul stand-in for the layer compute, and "
                         "print the hidden fraction of gather time as one JSON line")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--tokens", type=int, nargs="+", default=[512, 1024, 4096])
    ap.add_argument("--depths", type=int, nargs="+", default=[1, 2])
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Hot-path runner
# ---------------------------------------------------------------------------

class Runner:
    """One training step's ZeRO work on the workload, in the schedule of a
    stage ("ZeRO Stages: ...", stage sections):
      3: fused reduce-scatter + Adam, then each layer gathered before forward
         and again before backward (two gathers per step);
      2: the same reduction and update, then every rank's new slice is
         gathered back into the full copy that forward and backward read;
      1: the gradients all-reduced -- reduce-scatter into the accumulator,
         then its all-gather into a full fp32 gradient replica -- Adam from
         each rank's received slice, then the parameter all-gather.
    With micro-batches, stages 2 and 3 add each micro-batch's reduced shard
    into a shard-sized running sum; stage 1 all-reduces once per step."""

    def __init__(self, w, device, stage=3, split=False):
        import torch
        import zero_sharded_mixed_pad_amd as zsp
        from zero_sharded_mixed_pad_amd import synth

        self.torch, self.zsp, self.synth = torch, zsp, synth
        self.w, self.dev, self.stage, self.split = w, device, stage, split
        if stage < 3 and w.rank_local >= 0:
            raise ValueError("stages 1 and 2 gather every rank's shard; the workload holds one")
        self.plan = zsp.partition(w.numel, w.n_d)
        S, nd = self.plan.S, w.n_d
        self.rank = zsp.ALL_RANKS if w.rank_local < 0 else w.rank_local
        n_state = S if w.rank_local >= 0 else nd * S
        f32, bf16 = torch.float32, torch.bfloat16
        self.master = torch.empty(n_state, dtype=f32, device=device)
        self.m = torch.empty(n_state, dtype=f32, device=device)
        self.v = torch.empty(n_state, dtype=f32, device=device)
        self.work = torch.empty(n_state, dtype=bf16, device=device)
        need_acc = w.micro_batches > 1 or stage == 1 or split
        self.acc = torch.empty(n_state, dtype=f32, device=device) if need_acc else None
        # stage 1: every rank's full fp32 gradient after the all-reduce
        self.grad_replica = (torch.empty(self.plan.total_numel, dtype=f32, device=device)
                             if stage == 1 else None)
        self.plan.bind_state(self.rank, self.master, self.m, self.v, self.work, self.acc)
        flat = synth.flat_params(w, device=device)
        self.plan.load_params(flat)
        torch.cuda.synchronize()
        del flat
        self.layout = "shard" if w.rank_local >= 0 else "full"
        gsize = S if w.rank_local >= 0 else self.plan.total_padded
        self.grads = [synth.grad_buffer(w, gsize, r, device=device) for r in range(nd)]
        # valid (non-pad) elements the step updates
        if w.rank_local >= 0:
            j = w.rank_local
            self.valid = 0
            for t in range(len(w.numel)):
                s = self.plan.tensor(t)["shard_len"]
                self.valid += max(0, min(s, w.numel[t] - j * s))
        else:
            self.valid = self.plan.total_numel
        gb = 2 if w.grad_dtype == bf16 else 4
        acc_read = 4 if w.micro_batches > 1 else 0
        self.bytes_fused = self.valid * (nd * gb + 26 + acc_read)
        self.bytes_reduce_first = self.valid * (nd * gb + 4)
        self.bytes_reduce_acc = self.valid * (nd * gb + 8)
        self.bytes_adam = self.valid * (4 + 26)          # Adam from the accumulator
        self.bytes_gather_acc = self.valid * 8           # fp32 read + write
        # gathers: one per layer-sized group, before forward and before backward
        self.gather_groups = []
        if w.rank_local < 0:
            if w.name.startswith("mlp"):
                groups = [(t, 1) for t in range(len(w.numel))]
            else:
                groups = [(0, len(w.numel))]
            for first, n in groups:
                cnt = sum(w.numel[first:first + n])
                out = torch.empty(cnt, dtype=bf16, device=device)
                self.gather_groups.append((first, n, out, cnt * 4))
        self.step_no = 0
        self.open_event = None  # the end event of the last timed launch
        self.ev = {k: [] for k in STEP_KINDS + ("gather_cold", "gather_list",
                                                 "gather_list_cold", "gather_many_cold")}

    def _event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def _timed(self, kind, fn, record):
        """Run one launch. With `record`, time it from the event that
        closed the previous timed launch of the same sequence (or a new event
        when none is open) to an event recorded after it: consecutive
        launches share one event, so the markers between them add as little
        as they can to the step being timed."""
        if not record:
            fn()
            return
        if self.open_event is None:
            self.open_event = self._event()
            self.open_event.record()
        fn()
        b = self._event()
        b.record()
        self.ev[kind].append((self.open_event, b))
        self.open_event = b

    def step(self, record=False, start=None):
        """One step; with `record`, its launches are timed from `start` (an
        event already recorded) on, and open_event is left at the end of the
        last one."""
        w, p = self.w, self.plan
        self.step_no += 1
        self.open_event = start
        hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, step=self.step_no)
        if self.stage == 1:
            self._timed("reduce_set", lambda: p.reduce_shard(
                self.rank, self.grads, layout=self.layout, accumulate=False), record)
            self._timed("gather_acc", lambda: p.gather_range(
                0, len(w.numel), self.grad_replica, "acc"), record)
            self._timed("adam", lambda: p.adam_step(self.rank, **hp), record)
            for first, n, out, _b in self.gather_groups:
                self._timed("gather", lambda first=first, n=n, out=out: p.gather_range(
                    first, n, out, "work"), record)
            return
        if self.split:  # unfused: reduce into the accumulator, then Adam from it
            for mb in range(w.micro_batches):
                self._timed("reduce_acc" if mb > 0 else "reduce_set", lambda mb=mb: p.reduce_shard(
                    self.rank, self.grads, layout=self.layout, accumulate=mb > 0), record)
            self._timed("adam", lambda: p.adam_step(self.rank, **hp), record)
        elif w.micro_batches > 1:
            for mb in range(w.micro_batches - 1):
                self._timed("reduce_acc" if mb > 0 else "reduce_set", lambda mb=mb: p.reduce_shard(
                    self.rank, self.grads, layout=self.layout, accumulate=mb > 0), record)
            self._timed("fused", lambda: p.reduce_adam_step(
                self.rank, self.grads, layout=self.layout, use_acc=True, **hp), record)
        else:
            self._timed("fused", lambda: p.reduce_adam_step(
                self.rank, self.grads, layout=self.layout, **hp), record)
        # stage 3: before forward, and again before backward; stage 2: once,
        # after the update
        for _ in range(2 if self.stage == 3 else 1):
            for first, n, out, _b in self.gather_groups:
                self._timed("gather", lambda first=first, n=n, out=out: p.gather_range(
                    first, n, out, "work"), record)

    def cold_gathers(self, flush, reps):
        """Each gather group again, `reps` times, each time right after
        `flush` has evicted the caches: a gather under 1 GB can otherwise
        read what the step just wrote from the 256 MB Infinity Cache."""
        for _ in range(reps):
            for first, n, out, _b in self.gather_groups:
                flush()
                self.open_event = None
                self._timed("gather_cold", lambda first=first, n=n, out=out:
                            self.plan.gather_range(first, n, out, "work"), True)

    def list_gathers(self, flush, reps):
        """Every parameter at once, each into its own output, `reps` times:
        as a prepared list (zsp_gather_list_run: one launch over records
        built once) and, when `flush` is given, also as the one-shot call
        (zsp_gather_many: checks, staging and the record kernel each call).
        After `flush` they are recorded as gather_list_cold and
        gather_many_cold, beside the range form's gather_cold; without one,
        prepared runs back to back (gather_list)."""
        torch = self.torch
        from zero_sharded_mixed_pad_amd import binding
        if not hasattr(self, "glist"):
            ids = list(range(len(self.w.numel)))
            outs = [torch.empty(max(n, 1), dtype=torch.bfloat16, device=self.dev)
                    for n in self.w.numel]
            self.glist = self.plan.gather_list(ids, outs, "work")
            # marshalled once: the timed calls are the library's alone
            self.gmany = binding._list_arrays(ids, outs, torch.bfloat16)
        kind = "gather_list_cold" if flush else "gather_list"
        self.open_event = None
        for _ in range(reps):
            if flush:
                flush()
                self.open_event = None
            self._timed(kind, lambda: self.plan.gather_prepared(self.glist), True)
        if flush:
            ids_c, outs_c, n = self.gmany
            h, st = self.plan.handle, binding._stream(None)
            call = lambda: binding._check(binding.lib.zsp_gather_many(  # noqa: E731
                h, ids_c, n, binding.SRC_WORK, outs_c, st))
            for _ in range(reps):
                flush()
                self.open_event = None
                self._timed("gather_many_cold", call, True)

    def step_bytes(self):
        w = self.w
        gathers = sum(g[3] for g in self.gather_groups)
        if self.stage == 1:
            return self.bytes_reduce_first + self.bytes_gather_acc + self.bytes_adam + gathers
        if self.split:
            b = (self.bytes_reduce_first + (w.micro_batches - 1) * self.bytes_reduce_acc
                 + self.bytes_adam)
        else:
            b = self.bytes_fused
            if w.micro_batches > 1:
                b += self.bytes_reduce_first + (w.micro_batches - 2) * self.bytes_reduce_acc
        b += (2 if self.stage == 3 else 1) * gathers
        return b

    def bytes_of(self, kind):
        """Algorithmic bytes one launch of `kind` moves."""
        if kind == "fused":
            return self.bytes_fused
        if kind == "reduce_set":
            return self.bytes_reduce_first
        if kind == "reduce_acc":
            return self.bytes_reduce_acc
        if kind == "adam":
            return self.bytes_adam
        if kind == "gather_acc":
            return self.bytes_gather_acc
        if kind.startswith("gather_list") or kind == "gather_many_cold":
            return sum(g[3] for g in self.gather_groups)
        return sum(g[3] for g in self.gather_groups) / len(self.gather_groups)

    def trace_name(self, kind):
        """The kernel's name in the rocprofv3 summaries (bench.py --rocprof-summary)."""
        gdt = "bf16" if self.w.grad_dtype == self.torch.bfloat16 else "f32"
        if kind == "fused":
            acc = "_acc" if self.w.micro_batches > 1 and not self.split else ""
            return f"fused_reduce_adam_cast{acc}[{gdt}]"
        if kind in ("reduce_set", "reduce_acc"):
            return f"{kind}[{gdt}]"
        if kind == "adam":
            return "adam_from_acc[f32]"
        if kind == "gather_acc":
            return "gather[f32]"
        if kind.startswith("gather_list") or kind == "gather_many_cold":
            staged = sum(1 for n in self.w.numel if n > 0) > 64
            return f"gather_list_{'recs' if staged else 'args'}[bf16]"
        return "gather[bf16]"

    def kernel_stats(self, steps):
        """Per kind of launch: HIP-event times over the timed steps, the
        algorithmic bytes of one launch and the rate they give; for the kinds
        of the step, launches per step and the time per step they take."""
        out = {}
        for kind, evs in self.ev.items():
            if not evs:
                continue
            ms = [a.elapsed_time(b) for a, b in evs]
            avg_s = sum(ms) / len(ms) / 1e3
            nbytes = self.bytes_of(kind)
            gbps = nbytes / avg_s / 1e9
            srt = sorted(ms)
            med = (srt[(len(srt) - 1) // 2] + srt[len(srt) // 2]) / 2
            out[kind] = {"launches": len(ms), "avg_us": round(avg_s * 1e6, 2),
                         "median_us": round(med * 1e3, 2),
                         "min_us": round(min(ms) * 1e3, 2), "bytes_per_launch": int(nbytes),
                         "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                         "kernel": self.trace_name(kind)}
            if kind in STEP_KINDS:
                out[kind]["launches_per_step"] = round(len(ms) / steps, 3)
                out[kind]["us_per_step"] = round(avg_s * 1e6 * len(ms) / steps, 2)
        return out


def dominant_kind(ks):
    """The kind of launch that takes the most time per step."""
    kinds = [k for k in ks if k in STEP_KINDS]
    return max(kinds, key=lambda k: ks[k]["us_per_step"])


# ---------------------------------------------------------------------------
# Sharded checkpoint: save, load, load resharded
# ---------------------------------------------------------------------------

def checkpoint_bench(r, parent):
    """Wall time of zsp_checkpoint_save / zsp_checkpoint_load over every rank
    of the workload, after one real step, and of a load under N_d/2 ranks that
    rebuilds every shard from the saved ones. Loads are checked bit for bit
    (the resharded one by gathering every parameter from both plans)."""
    import shutil
    import tempfile
    torch, zsp, w = r.torch, r.zsp, r.w
    r.step()
    torch.cuda.synchronize()
    state = (r.master, r.m, r.v, r.work)
    before = [x.clone() for x in state]
    n_files = 1 if w.rank_local >= 0 else w.n_d
    file_bytes = n_files * (8 + 5 * 8 + 8 * len(w.numel) + 14 * r.plan.S + 8)
    d = tempfile.mkdtemp(prefix="zsp_ckpt_", dir=parent)
    out = {"dir_parent": parent, "files": n_files, "file_bytes": file_bytes}
    try:
        t = time.perf_counter()
        r.plan.checkpoint_save(r.rank, d, r.step_no)
        out["save_s"] = time.perf_counter() - t
        for x in state:
            x.zero_()
        torch.cuda.synchronize()
        t = time.perf_counter()
        step = r.plan.checkpoint_load(r.rank, d)
        out["load_s"] = time.perf_counter() - t
        assert step == r.step_no
        out["load_bit_exact"] = all(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16
                                                else a.view(torch.int32),
                                                b.view(torch.int16) if b.dtype == torch.bfloat16
                                                else b.view(torch.int32))
                                    for a, b in zip(state, before))
        del before
        if w.rank_local < 0 and w.n_d % 2 == 0:
            nd2 = w.n_d // 2
            p2 = zsp.partition(w.numel, nd2)
            n2 = nd2 * p2.S
            st2 = [torch.empty(n2, dtype=torch.float32, device=r.dev) for _ in range(3)]
            st2.append(torch.empty(n2, dtype=torch.bfloat16, device=r.dev))
            p2.bind_state(zsp.ALL_RANKS, *st2)
            torch.cuda.synchronize()
            t = time.perf_counter()
            p2.checkpoint_load(zsp.ALL_RANKS, d)
            out["reshard_load_s"] = time.perf_counter() - t
            out["reshard_to_n_d"] = nd2
            ok = True
            for first, n, buf, _b in r.gather_groups:
                a = torch.empty_like(buf)
                r.plan.gather_range(first, n, a, "work")
                p2.gather_range(first, n, buf, "work")
                ok = ok and torch.equal(a.view(torch.int16), buf.view(torch.int16))
            for src in ("master",):
                for t_ in range(len(w.numel)):
                    a = torch.empty(w.numel[t_], dtype=torch.float32, device=r.dev)
                    b = torch.empty_like(a)
                    r.plan.gather(t_, a, src)
                    p2.gather(t_, b, src)
                    ok = ok and torch.equal(a.view(torch.int32), b.view(torch.int32))
            torch.cuda.synchronize()
            out["reshard_bit_exact"] = bool(ok)
            p2.destroy()
            del st2
    finally:
        shutil.rmtree(d, ignore_errors=True)
    for k in ("save", "load", "reshard_load"):
        if k + "_s" in out:
            out[k + "_GBps"] = round(file_bytes / out[k + "_s"] / 1e9, 3)
            out[k + "_s"] = round(out[k + "_s"], 3)
    return out


# ---------------------------------------------------------------------------
# Per-layer gather schedule with prefetch
# ---------------------------------------------------------------------------

def prefetch_bench(args, device):
    """Forward (layers 0..L-1) then backward (L-1..0) over a Llama-7B decoder
    stack whose layers are gathered by zsp_sched_* into a (D+1)-slot arena.
    Per layer the compute stand-in runs the seven weight matmuls: forward
    Y = X W^T; backward dX = dY W and dW = dY^T X. Each pass is timed with
    events on the compute stream, whose last work waits for every gather.
    Modes are interleaved pass by pass over `steps` rounds (medians), since
    the hidden time is a small difference of large ones:

      compute  = passes on one fixed, already gathered layer (no gathers)
      gathers  = passes of gathers alone (depth 0, no compute)
      depth D  = gathers through the schedule with compute
      hidden(D) = (compute + gathers - depth D) / gathers
    each for the gather kernel and for the copy engines (copy_*).
    """
    import statistics
    import torch
    import zero_sharded_mixed_pad_amd as zsp
    from zero_sharded_mixed_pad_amd import synth

    w = synth.llama_stack(args.layers, 8)
    plan = zsp.partition(w.numel, w.n_d)
    n = w.n_d * plan.S
    state = [torch.empty(n, dtype=torch.float32, device=device) for _ in range(3)]
    state.append(torch.empty(n, dtype=torch.bfloat16, device=device))
    plan.bind_state(zsp.ALL_RANKS, *state)
    flat = synth.flat_params(w, device=device)
    plan.load_params(flat)
    torch.cuda.synchronize()
    del flat
    L = args.layers
    groups = [(9 * l, 9) for l in range(L)]
    order = list(range(L)) + list(range(L - 1, -1, -1))
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]  # (out, in)
    layer_elems = sum(w.numel[:9])
    cs, gs = torch.cuda.Stream(), torch.cuda.Stream()
    fixed = torch.empty(layer_elems, dtype=torch.bfloat16, device=device)
    plan.gather_range(0, 9, fixed, "work")
    fixed_views, k = [], 0
    for t in range(9):
        fixed_views.append(fixed[k:k + w.numel[t]])
        k += w.numel[t]
    scheds = {}
    for engine in ("kernel", "copy"):
        for D in [0] + list(args.depths):
            s = zsp.Schedule(plan, groups, order, D)
            s.set_engine(engine)
            arena = torch.empty(s.arena_bytes, dtype=torch.uint8, device=device)
            s.bind(arena, gs if D > 0 else None)
            scheds[(engine, D)] = (s, arena)
    torch.cuda.synchronize()

    results = {"layers": L, "n_d": w.n_d, "positions": len(order),
               "gather_bytes_per_layer": 4 * layer_elems,
               "arena_bytes": {str(D): s.arena_bytes for (e, D), (s, _a) in scheds.items()
                               if e == "kernel"},
               "runs": []}
    for T in args.tokens:
        x = {d: torch.randn(T, d, device=device, dtype=torch.bfloat16) * 0.1
             for d in (4096, 11008)}
        dw = {sh: torch.empty(sh, device=device, dtype=torch.bfloat16) for sh in set(shapes)}

        def compute(views, backward):
            for v, (o, i) in zip(views[:7], shapes):
                W = v.view(o, i)
                if not backward:
                    torch.nn.functional.linear(x[i], W)
                else:
                    dy = x[o]
                    torch.mm(dy, W)
                    torch.mm(dy.t(), x[i], out=dw[(o, i)])

        def one_pass(sched, with_compute):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(cs):
                a.record(cs)
                for p in range(len(order)):
                    if sched is None:
                        compute(fixed_views, p >= L)
                        continue
                    views = sched.acquire(p, cs)
                    if with_compute:
                        compute(views, p >= L)
                    sched.release(p, cs)
                b.record(cs)
            return a, b

        modes = [("compute", None, True), ("gathers", scheds[("kernel", 0)][0], False),
                 ("gathers_copy", scheds[("copy", 0)][0], False)]
        modes += [(f"depth{D}", scheds[("kernel", D)][0], True) for D in [0] + list(args.depths)]
        modes += [(f"copy_depth{D}", scheds[("copy", D)][0], True)
                  for D in [0] + list(args.depths)]
        for _ in range(max(1, args.warmup)):
            for _name, sch, wc in modes:
                one_pass(sch, wc)
        torch.cuda.synchronize()
        evs = {name: [] for name, _s, _w in modes}
        for _ in range(args.steps):
            for name, sch, wc in modes:
                evs[name].append(one_pass(sch, wc))
        torch.cuda.synchronize()
        ms = {name: statistics.median(a.elapsed_time(b) for a, b in e) for name, e in evs.items()}
        c, g, gc = ms["compute"], ms["gathers"], ms["gathers_copy"]
        row = {"tokens": T, "compute_ms": round(c, 3), "gathers_ms": round(g, 3),
               "gather_GBps": round(4 * layer_elems * len(order) / g / 1e6, 1),
               "copy_gathers_ms": round(gc, 3),
               "copy_gather_GBps": round(4 * layer_elems * len(order) / gc / 1e6, 1),
               "depth": {}, "copy_depth": {}}
        for D in [0] + list(args.depths):
            t = ms[f"depth{D}"]
            row["depth"][str(D)] = {"ms": round(t, 3), "exposed_gather_ms": round(t - c, 3),
                                    "hidden": round((c + g - t) / g, 3)}
            t = ms[f"copy_depth{D}"]
            row["copy_depth"][str(D)] = {"ms": round(t, 3), "exposed_gather_ms": round(t - c, 3),
                                         "hidden": round((c + gc - t) / gc, 3)}
        results["runs"].append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del x, dw
    for s, _a in scheds.values():
        s.destroy()
    plan.destroy()
    return results


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def cpu_model():
    """The host CPU's model name as /proc/cpuinfo reports it, or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def software():
    """Versions the measurement ran on."""
    import torch
    return {"torch": torch.__version__, "hip": torch.version.hip,
            "gpu": torch.cuda.get_device_name(0) if torch.cuda.is_available() else None}


# Rank j's real elements in the oracle sample: parameters are taken from the
# first one on until they reach this count (or the model ends).
CPU_SAMPLE_ELEMS = 8 << 20


def cpu_sample(runner, limit=CPU_SAMPLE_ELEMS):
    """Host copies of one virtual rank's share of the workload: its slices of
    the first parameters (together at least `limit` of its real elements, or
    every parameter), cut from the device buffers on the device so that only
    the sample crosses to the host. A prefix of the parameter list has the
    same per-parameter layout (pad, shard length, offsets) on its own as
    inside the whole list, so the oracle runs on that prefix as a model of
    its own. Returns the prefix, the rank, its gradient chunks in shard
    layout (the slice each rank sends to it), its state, and every rank's
    working copy of the prefix (for the gathers; None if rank-local)."""
    import numpy as np
    import torch
    import oracle

    w, nd = runner.w, runner.w.n_d
    L = oracle.Layout(w.numel, nd)
    j = w.rank_local if w.rank_local >= 0 else 0
    b, got = 0, 0
    while b < L.T and (b == 0 or got < limit):
        s = int(L.shard_len[b])
        got += max(0, min(s, int(L.numel[b]) - j * s))
        b += 1
    sub = [int(n) for n in w.numel[:b]]
    Ss = int(L.shard_off[b])           # the prefix's S: shard_off is a prefix sum

    def host(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    torch.cuda.synchronize()
    grads = []
    for g in runner.grads:
        if w.rank_local >= 0:
            grads.append(host(g[:Ss]))
        else:
            parts = [g[int(L.full_off[t]) + j * int(L.shard_len[t]):
                       int(L.full_off[t]) + (j + 1) * int(L.shard_len[t])] for t in range(b)]
            grads.append(host(torch.cat(parts)))
    base = 0 if w.rank_local >= 0 else j * L.S
    state = [host(x[base:base + Ss]).copy() for x in (runner.master, runner.m, runner.v,
                                                       runner.work)]
    all_work = None
    if w.rank_local < 0:
        all_work = host(torch.cat([runner.work[r * L.S:r * L.S + Ss] for r in range(nd)]))
    valid = int(sum(max(0, min(int(L.shard_len[t]), int(L.numel[t]) - j * int(L.shard_len[t])))
                    for t in range(b)))
    return sub, j, grads, state, all_work, valid


def cpu_baseline(runner, target_s):
    """The oracle as it stands, timed on the host on a bounded sample of the
    workload (cpu_sample): one virtual rank's reduce over the N_d gradient
    chunks + Adam + cast on its slices of the first parameters, plus the
    gathers of those parameters. Measured twice for about target_s each: on
    one thread, and on one thread per host core of the process's CPU share
    (at most 16), each thread updating its own copy of the rank's state (the
    oracle's C calls release Python's lock)."""
    import threading

    import torch
    import oracle

    w = runner.w
    nd = w.n_d
    sub, j, grads, state0, all_work, valid = cpu_sample(runner)
    gb = 2 if w.grad_dtype == torch.bfloat16 else 4
    T = len(sub)

    def worker(gather_ids, out):
        master, m, v, work = (x.copy() for x in state0)
        fused_bytes = valid * (nd * gb + 26)
        gather_bytes = sum(sub[t] * 4 for t in gather_ids)
        done, passes, t0 = 0, 0, time.perf_counter()
        while True:
            red = oracle.reduce(sub, nd, j, grads, oracle.GRADS_SHARD)
            oracle.adam(sub, nd, j, master, m, v, work, red, w.lr, w.beta1, w.beta2, w.eps,
                        passes + 1)
            for t in gather_ids:
                oracle.gather(sub, nd, t, all_work)
            done += fused_bytes + gather_bytes
            passes += 1
            el = time.perf_counter() - t0
            if el >= target_s or el * (passes + 1) / passes > 3 * target_s:
                break
        out.append((done, passes))

    def run(threads):
        gathers = [[t for t in range(T) if t % threads == i] if all_work is not None else []
                   for i in range(threads)]
        outs = [[] for _ in range(threads)]
        ts = [threading.Thread(target=worker, args=(gathers[i], outs[i]))
              for i in range(threads)]
        t0 = time.perf_counter()
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        el = time.perf_counter() - t0
        return sum(o[0][0] for o in outs) / el / 1e9, el, min(o[0][1] for o in outs)

    one, el1, p1 = run(1)
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    threads = max(1, min(16, share))
    many, eln, pn = run(threads) if threads > 1 else (one, el1, p1)
    what = (f"each thread: virtual rank {j}'s reduce over {nd} gradient chunks + Adam + cast "
            f"on its own copy of rank {j}'s state, for parameters 0..{T - 1} of {len(w.numel)} "
            f"({valid} of the rank's real elements)"
            + ("" if all_work is None else
               f", plus the gathers of its share of those {T} parameters"))
    return {"value": round(many, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "seconds": round(eln, 2),
            "sample": f"{what}; at least {pn} pass(es) per thread (C oracle, unchanged)",
            "single_core": {"value": round(one, 3), "cores": 1, "seconds": round(el1, 2),
                            "passes": p1}}


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------

_OPS = {0: "copy_in", 1: "reduce_set", 2: "reduce_acc", 3: "fused_reduce_adam_cast",
        4: "fused_reduce_adam_cast_acc", 5: "adam_from_acc"}


def _short(name):
    """Readable kernel name from a mangled or demangled rocprofv3 name."""
    import re
    m = re.search(r"shard_kernel(?:ILi|<)(\d)", name)
    if m:
        dt = "f32" if ("ILi%sEf" % m.group(1)) in name or ", float" in name else "bf16"
        return f"{_OPS[int(m.group(1))]}[{dt}]"
    if "gather_kernel" in name:
        return "gather[f32]" if ("IfE" in name or "<float>" in name) else "gather[bf16]"
    if "gather_span_kernel" in name:  # the range gather's form over short pieces (bf16)
        return "gather[bf16]"
    m = re.search(r"gather_list_(args|recs)", name)
    if m:
        dt = "f32" if ("IfLb" in name or "<float," in name) else "bf16"
        return f"gather_list_{m.group(1)}[{dt}]"
    if "list_expand_kernel" in name:
        return "gather_list_expand"
    name = re.sub(r"^void ", "", name)
    return name[:48]


def rocprof_summary(d, out):
    lines = []
    stats = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    for path in stats:
        lines.append(f"kernel stats: {os.path.relpath(path, d)}")
        lines.append(f"{'kernel':<48} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}")
        with open(path) as f:
            for row in csv.DictReader(f):
                lines.append(f"{_short(row['Name']):<48} {row['Calls']:>6} "
                             f"{float(row['AverageNs']) / 1e3:>10.2f} "
                             f"{float(row['MinNs']) / 1e3:>10.2f} "
                             f"{float(row['MaxNs']) / 1e3:>10.2f}")
    counters = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    for path in counters:
        agg = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                k = (_short(row["Kernel_Name"]), row["Counter_Name"])
                agg.setdefault(k, []).append(float(row["Counter_Value"]))
        lines.append(f"counters: {os.path.relpath(path, d)}")
        lines.append(f"{'kernel':<48} {'counter':<12} {'dispatches':>10} {'avg_KiB':>14}")
        for (k, c), vals in sorted(agg.items()):
            lines.append(f"{k:<48} {c:<12} {len(vals):>10} {sum(vals) / len(vals):>14.1f}")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


def _counter_rows(d, counter):
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    rows.append((row["Kernel_Name"], float(row["Counter_Value"])))
    return rows


def traffic_from(fetch_dir, write_dir, workload):
    """HBM bytes per launch of the fused and gather kernels from PMC counters.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by the
    factor that maps the same counter onto a plain 2 GiB device copy's known
    2 GiB of reads and 2 GiB of writes."""
    copy_bytes = float(2 << 30)
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "calibration": "torch copy_ of a 2 GiB bf16 tensor: 2 GiB read, 2 GiB written"}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copies = [v for n, v in rows if "copy" in n.lower() or "elementwise" in n.lower()]
        copies = [v for v in copies if v * 1024 > 0.5 * copy_bytes]
        if not copies:
            raise SystemExit(f"no calibration copy found among {counter} dispatches")
        factor = copy_bytes / (sum(copies) / len(copies) * 1024)
        out[f"{counter}_copy_KiB"] = round(sum(copies) / len(copies), 1)
        out[f"{counter}_factor"] = round(factor, 4)
        for n, v in rows:
            k = _short(n)
            per.setdefault(k, {}).setdefault(counter, []).append(v * 1024 * factor)
    for k, d in per.items():
        if "FETCH_SIZE" in d and "WRITE_SIZE" in d and not k.startswith("at::"):
            f = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"])
            w = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"])
            out.setdefault("kernels", {})[k] = {"read_bytes": int(f), "write_bytes": int(w),
                                                "bytes_per_launch": int(f + w),
                                                "dispatches": len(d["FETCH_SIZE"])}
    fused = [v for k, v in out.get("kernels", {}).items() if k.startswith("fused_reduce_adam_cast")]
    out["fused_bytes_per_launch"] = fused[0]["bytes_per_launch"] if fused else None
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def load_traffic(workload, kernel):
    """Measured HBM bytes per launch of `kernel` (its name in the rocprofv3
    summaries) from the committed counter summary of `workload`, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return k["bytes_per_launch"] if k else None


# ---------------------------------------------------------------------------

def time_workload(w, args, device, evict, say):
    """Build the workload's runner, run `warmup` untimed steps and time
    `steps` steps. Returns the runner and the workload's figures."""
    import torch
    say(f"[bench] {w.name}: setting up")
    r = Runner(w, device, args.stage, args.split)
    flush = args.flush == "on" or (args.flush == "auto" and r.bytes_fused < 2e9)
    for _ in range(args.warmup):
        if flush:
            evict()
        r.step()
    torch.cuda.synchronize()
    step_events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if flush:
            evict()
        a = torch.cuda.Event(enable_timing=True)
        a.record()
        r.step(record=True, start=a)
        step_events.append((a, r.open_event))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms = sum(a.elapsed_time(b) for a, b in step_events) / args.steps
    # Without a flush the wall clock around the K steps is the step time; with
    # one, the per-step events exclude the flush kernel.
    ms_per_step = event_ms if flush else wall * 1e3 / args.steps
    step_bytes = r.step_bytes()
    value = step_bytes / (ms_per_step / 1e3) / 1e9
    if not flush and any(g[3] < 1e9 for g in r.gather_groups):
        r.cold_gathers(evict, args.steps)
        torch.cuda.synchronize()
    if r.gather_groups and args.stage == 3:
        cold = sum(g[3] for g in r.gather_groups) < 1e9
        r.list_gathers(evict if cold else None, args.steps)
        torch.cuda.synchronize()
    ks = r.kernel_stats(args.steps)
    dom = dominant_kind(ks)
    fig = {"ms_per_step": round(ms_per_step, 4), "GBps": round(value, 1),
           "frac_hbm_peak": round(value / HBM_PEAK_GBPS, 4), "bytes_per_step": int(step_bytes),
           "wall_ms_per_step": round(wall * 1e3 / args.steps, 4), "cache_flush": bool(flush),
           "dominant": dom, "kernels": ks}
    say(f"[bench] {w.name}: {ms_per_step:.3f} ms/step, {value:.1f} GB/s; dominant {dom} "
        f"{ks[dom]['GBps']} GB/s ({ks[dom]['frac_hbm_peak']})")
    return r, fig


def roofline(r, w, fig):
    """Roofline object for the kind of launch that takes the most time per
    step, with the whole step's fraction of peak beside it."""
    ks, dom = fig["kernels"], fig["dominant"]
    k = ks[dom]
    name = r.trace_name(dom)
    roof = {"bound": "hbm", "achieved": k["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(k["GBps"] / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(w.name, name),
            "kernel": name, "kind": dom,
            "launches_per_step": k["launches_per_step"],
            "bytes_per_launch": k["bytes_per_launch"], "avg_launch_us": k["avg_us"],
            "step_frac": fig["frac_hbm_peak"]}
    # counter-measured HBM bytes (FETCH_SIZE + WRITE_SIZE) over the same launch time
    roof["traffic_GBps"] = (round(roof["traffic"] / k["avg_us"] / 1e3, 1)
                            if roof["traffic"] and k["avg_us"] else None)
    return roof


def main():
    args = parse()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary, args.summary_out)
        return 0
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import __graft_entry__
    __graft_entry__.ensure_built()
    import torch
    from zero_sharded_mixed_pad_amd import synth

    def say(msg):
        print(msg, file=sys.stderr, flush=True)

    wl = synth.workloads()
    if args.workload not in wl:
        print(f"unknown workload {args.workload}; choose from {sorted(wl)}", file=sys.stderr)
        return 2
    w = wl[args.workload]
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.prefetch:
        res = prefetch_bench(args, device)
        print(json.dumps({"mode": "prefetch", "steps": args.steps, "warmup": args.warmup,
                          **res}), flush=True)
        return 0
    if args.checkpoint:
        r = Runner(w, device, args.stage, args.split)
        res = checkpoint_bench(r, args.checkpoint)
        print(json.dumps({"mode": "checkpoint", "workload": w.name, "n_d": w.n_d, **res}),
              flush=True)
        return 0
    # Cache flush: a reduction that reads 1 GiB, four times the Infinity
    # Cache, evicting the working set without leaving dirty lines behind (a
    # flush that writes would make the timed kernel pay their write-back).
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=device)
    sink = torch.empty((), dtype=torch.float32, device=device)

    def evict():
        torch.sum(scratch, dim=0, out=sink)

    r, fig = time_workload(w, args, device, evict, say)
    roof = roofline(r, w, fig)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.bfloat16, device=device)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        say("[bench] CPU oracle baseline")
        cpu = cpu_baseline(r, args.cpu_seconds)
        cpu["value_vs_gpu_ratio"] = round(fig["GBps"] / cpu["value"], 1) if cpu["value"] else None

    gdt = "bf16" if w.grad_dtype == torch.bfloat16 else "f32"
    pdt = "bf16" if w.param_dtype == torch.bfloat16 else "f32"
    config = {"workload": w.name, "n_d": w.n_d, "params": len(w.numel),
              "elements": sum(w.numel), "param_dtype": pdt, "grad_dtype": gdt,
              "state": "fp32 master, m, v + bf16 working copy",
              "micro_batches": w.micro_batches,
              "rank_local": w.rank_local if w.rank_local >= 0 else None,
              "zero_stage": args.stage,
              "gathers_per_step": (2 if args.stage == 3 else 1) * len(r.gather_groups),
              "bytes_per_step": fig["bytes_per_step"], "cache_flush": fig["cache_flush"],
              "wall_ms_per_step": fig["wall_ms_per_step"]}
    ks = fig["kernels"]
    del r
    torch.cuda.empty_cache()

    # The other workloads, each timed the same way (per-kernel figures only).
    workloads = {w.name: {k: v for k, v in fig.items()}}
    if args.all_workloads:
        for name, ow in wl.items():
            if name == w.name:
                continue
            ro, ofig = time_workload(ow, args, device, evict, say)
            ofig["roofline_frac"] = round(ofig["kernels"][ofig["dominant"]]["frac_hbm_peak"], 4)
            workloads[name] = ofig
            del ro
            torch.cuda.empty_cache()
    workloads[w.name]["roofline_frac"] = roof["frac"]

    line = {
        "metric": METRIC, "value": fig["GBps"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": fig["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded normal gradients and parameters, resident in HBM)",
        "config": config, "roofline": roof, "cpu_baseline": cpu, "kernels": ks,
        "workloads": workloads,
        "kernel_source_hash": kernel_source_hash(), "software": software(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
