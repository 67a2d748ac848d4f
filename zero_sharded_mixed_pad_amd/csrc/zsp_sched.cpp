// zsp_sched.cpp -- the per-layer gather schedule of stage 3 with prefetch
// ("ZeRO Stage 3: Parameter Partitioning", the on-demand fetch list and the
// prefetch paragraph; "ZeRO Stages: Sharding Optimizer State, Gradients, and
// Parameters", "Stage 3 partitions parameters": each layer's parameters are
// gathered before its forward and again before its backward, released after
// use, and gathering one layer ahead hides the gather behind the current
// layer's arithmetic; the prefetch depth trades memory for exposed time).
//
// A schedule is a list of groups (consecutive parameter ranges, one layer
// each) and an order of positions over them (e.g. forward 0..L-1 then
// backward L-1..0). Position p gathers into slot p mod (D+1) of a
// caller-owned arena, D being the prefetch depth. Ordering is carried by
// HIP events only; the host never waits:
//   * gathers run on the caller's gather stream. Before issuing new gathers,
//     that stream waits on `mark`: the compute-stream point of the latest
//     release, or, at position 0, the point where the pass began. Position
//     p's acquire issues the gather of position p+D into the slot that
//     position p-1 used, so waiting for p-1's release is exactly the slot's
//     reuse condition; at position 0 it orders the pass's gathers after the
//     optimizer step that precedes it on the compute stream.
//   * the compute stream waits on the slot's `got` event before the caller's
//     work on position p.
// Depth 0 gathers on the compute stream itself, in line: the gather-then-
// compute baseline with nothing hidden.
//
// Gathers run either as the gather kernel (the default) or on the DMA copy
// engines (ZSP_ENGINE_COPY): one device-to-device copy that uses no compute
// units per rank's slice of each parameter, in order on the same stream the
// kernel would run on, so the same events order them.
#include <algorithm>
#include <new>
#include <vector>

#include "zsp_entry.hpp"
#include "zsp_internal.hpp"
#include "zsp_plan.hpp"

namespace {

constexpr int32_t kMaxDepth = 64;

int64_t round_up256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace

struct zsp_sched {
    zsp_plan* plan = nullptr;
    std::vector<int32_t> first, count;  // per group: consecutive parameters
    std::vector<int32_t> order;         // group of each position
    int32_t depth = 0;
    int32_t slots = 1;
    zsp_source src = ZSP_SRC_WORK;
    int64_t slot_bytes = 0;
    zsp_gather_engine engine = ZSP_ENGINE_KERNEL;

    bool bound = false;
    int device = -1;
    char* arena = nullptr;
    hipStream_t gstream = nullptr;
    std::vector<hipEvent_t> got;  // per slot: its latest gather has finished
    hipEvent_t mark = nullptr;    // compute-stream point new gathers must follow

    int32_t next = 0;     // position the next acquire must name
    int32_t held = -1;    // acquired and not yet released, or -1
    int32_t issued = -1;  // last position of this pass whose gather is issued
};

namespace {

void drop_events(zsp_sched* s) {
    for (hipEvent_t e : s->got)
        if (e) (void)hipEventDestroy(e);
    s->got.clear();
    if (s->mark) (void)hipEventDestroy(s->mark);
    s->mark = nullptr;
}

void* slot_ptr(const zsp_sched* s, int32_t pos) {
    return s->arena + int64_t(pos % s->slots) * s->slot_bytes;
}

// Copy-engine gather of position pos's group, in order on `stream`.
zsp_status copy_gather(zsp_sched* s, int32_t pos, hipStream_t stream) {
    const zsp_plan* P = s->plan;
    zsp_status st = zsp::check_bound(P);
    if (st != ZSP_OK) return st;
    if (P->bind_rank != ZSP_ALL_RANKS)
        return zsp::set_error(ZSP_ESTATE, "gather needs every rank's shard");
    const int32_t g = s->order[size_t(pos)];
    const int32_t f = s->first[size_t(g)], c = s->count[size_t(g)];
    const int64_t esz = s->src == ZSP_SRC_WORK ? 2 : 4;
    const char* src = s->src == ZSP_SRC_WORK ? reinterpret_cast<const char*>(P->work)
                                             : reinterpret_cast<const char*>(P->master);
    char* out = static_cast<char*>(slot_ptr(s, pos));
    for (int32_t t = f; t < f + c; ++t) {
        const int64_t sl = P->shard_len[size_t(t)], n = P->numel[size_t(t)];
        const int64_t o = P->flat_off[size_t(t)] - P->flat_off[size_t(f)];
        for (int32_t r = 0; r < P->nd && int64_t(r) * sl < n; ++r) {
            const int64_t cnt = std::min(sl, n - int64_t(r) * sl);
            const hipError_t e =
                hipMemcpyAsync(out + (o + int64_t(r) * sl) * esz,
                               src + (int64_t(r) * P->S + P->shard_off[size_t(t)]) * esz,
                               size_t(cnt * esz), hipMemcpyDeviceToDeviceNoCU, stream);
            if (e != hipSuccess) return zsp::set_hip_error(e, "copy-engine gather");
        }
    }
    return ZSP_OK;
}

zsp_status issue_gather(zsp_sched* s, int32_t pos, hipStream_t stream) {
    if (s->engine == ZSP_ENGINE_COPY) return copy_gather(s, pos, stream);
    const int32_t g = s->order[size_t(pos)];
    return zsp::gather_range(s->plan, s->first[size_t(g)], s->count[size_t(g)], s->src,
                             slot_ptr(s, pos), stream);
}

}  // namespace

extern "C" {

zsp_status zsp_sched_create(zsp_plan* plan, int32_t n_groups, const int32_t* group_first,
                            const int32_t* group_count, int32_t n_steps, const int32_t* order,
                            int32_t depth, zsp_source src, int64_t* arena_bytes,
                            zsp_sched** out) {
    using zsp::set_error;
    if (!out) return set_error(ZSP_EINVAL, "out is NULL");
    *out = nullptr;
    if (!plan) return set_error(ZSP_EINVAL, "plan is NULL");
    if (!arena_bytes) return set_error(ZSP_EINVAL, "arena_bytes is NULL");
    if (n_groups < 1 || !group_first || !group_count)
        return set_error(ZSP_EINVAL, "need at least one group (n_groups=%d)", n_groups);
    if (n_steps < 1 || !order) return set_error(ZSP_EINVAL, "need at least one position");
    if (depth < 0 || depth > kMaxDepth)
        return set_error(ZSP_EINVAL, "prefetch depth %d outside [0, %d]", depth, kMaxDepth);
    if (src != ZSP_SRC_WORK && src != ZSP_SRC_MASTER)
        return set_error(ZSP_EINVAL, "bad source %d", src);
    const int64_t esize = src == ZSP_SRC_WORK ? 2 : 4;
    int64_t largest = 0;
    for (int32_t g = 0; g < n_groups; ++g) {
        const int32_t f = group_first[g], c = group_count[g];
        if (c < 1 || f < 0 || f > plan->T - c)
            return set_error(ZSP_ERANGE, "group %d: parameters [%d, %d+%d) outside [0, %d)", g, f,
                             f, c, plan->T);
        largest = std::max(largest, plan->flat_off[size_t(f + c)] - plan->flat_off[size_t(f)]);
    }
    for (int32_t p = 0; p < n_steps; ++p)
        if (order[p] < 0 || order[p] >= n_groups)
            return set_error(ZSP_ERANGE, "position %d names group %d outside [0, %d)", p,
                             order[p], n_groups);
    zsp_sched* s = new (std::nothrow) zsp_sched;
    if (!s) return set_error(ZSP_ENOMEM, "out of host memory");
    try {
        s->first.assign(group_first, group_first + n_groups);
        s->count.assign(group_count, group_count + n_groups);
        s->order.assign(order, order + n_steps);
    } catch (const std::bad_alloc&) {
        delete s;
        return set_error(ZSP_ENOMEM, "out of host memory");
    }
    s->plan = plan;
    s->depth = std::min(depth, n_steps - 1);
    s->slots = s->depth + 1;
    s->src = src;
    s->slot_bytes = round_up256(std::max<int64_t>(largest * esize, 1));
    *arena_bytes = s->slot_bytes * s->slots;
    *out = s;
    return ZSP_OK;
}

zsp_status zsp_sched_bind(zsp_sched* s, void* arena, int64_t arena_bytes, void* gather_stream) {
    using zsp::set_error;
    if (!s) return set_error(ZSP_EINVAL, "schedule is NULL");
    zsp_plan* P = s->plan;
    if (!P->bound || P->bind_rank != ZSP_ALL_RANKS)
        return set_error(ZSP_ESTATE, "the plan must have every rank's state bound");
    if (!arena || (reinterpret_cast<uintptr_t>(arena) & 255u) != 0)
        return set_error(ZSP_EINVAL, "arena is NULL or not 256-byte aligned");
    if (arena_bytes < s->slot_bytes * s->slots)
        return set_error(ZSP_ERANGE, "arena holds %lld bytes; the schedule needs %lld",
                         (long long)arena_bytes, (long long)(s->slot_bytes * s->slots));
    if (s->depth > 0 && !gather_stream)
        return set_error(ZSP_EINVAL, "prefetch needs a gather stream of its own");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return zsp::set_hip_error(e, "hipGetDevice");
    if (dev != P->device)
        return set_error(ZSP_ESTATE, "plan is bound on device %d but device %d is current",
                         P->device, dev);
    drop_events(s);
    s->bound = false;
    if (s->depth > 0) {
        s->got.assign(size_t(s->slots), nullptr);
        for (hipEvent_t& ev : s->got) {
            if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
                drop_events(s);
                return zsp::set_hip_error(e, "hipEventCreateWithFlags");
            }
        }
        if ((e = hipEventCreateWithFlags(&s->mark, hipEventDisableTiming)) != hipSuccess) {
            drop_events(s);
            return zsp::set_hip_error(e, "hipEventCreateWithFlags");
        }
    }

    s->arena = static_cast<char*>(arena);
    s->gstream = static_cast<hipStream_t>(gather_stream);
    s->device = dev;
    s->bound = true;
    s->next = 0;
    s->held = -1;
    s->issued = -1;
    return ZSP_OK;
}

zsp_status zsp_sched_acquire(zsp_sched* s, int32_t position, void* compute_stream,
                             void** params) {
    using zsp::set_error;
    if (!s) return set_error(ZSP_EINVAL, "schedule is NULL");
    if (!params) return set_error(ZSP_EINVAL, "params is NULL");
    if (!s->bound) return set_error(ZSP_ESTATE, "schedule has no arena (call zsp_sched_bind)");
    if (s->held >= 0)
        return set_error(ZSP_ESTATE, "position %d is still held (release it first)", s->held);
    if (position != s->next)
        return set_error(ZSP_ESTATE, "acquire of position %d out of order (expected %d)",
                         position, s->next);
    hipStream_t cs = static_cast<hipStream_t>(compute_stream);
    zsp_status st;
    if (s->depth == 0) {
        if ((st = issue_gather(s, position, cs)) != ZSP_OK) return st;
    } else {
        const int32_t last = std::min<int32_t>(position + s->depth, int32_t(s->order.size()) - 1);
        hipError_t e = hipSuccess;
        if (position == 0) e = hipEventRecord(s->mark, cs);
        if (e == hipSuccess && last > s->issued) e = hipStreamWaitEvent(s->gstream, s->mark, 0);
        if (e != hipSuccess) return zsp::set_hip_error(e, "ordering the gather stream");
        for (int32_t q = s->issued + 1; q <= last; ++q) {
            if ((st = issue_gather(s, q, s->gstream)) != ZSP_OK) return st;
            if ((e = hipEventRecord(s->got[size_t(q % s->slots)], s->gstream)) != hipSuccess)
                return zsp::set_hip_error(e, "hipEventRecord");
            s->issued = q;
        }
        if ((e = hipStreamWaitEvent(cs, s->got[size_t(position % s->slots)], 0)) != hipSuccess)
            return zsp::set_hip_error(e, "ordering the compute stream");
    }
    s->held = position;
    *params = slot_ptr(s, position);
    return ZSP_OK;
}

zsp_status zsp_sched_release(zsp_sched* s, int32_t position, void* compute_stream) {
    using zsp::set_error;
    if (!s) return set_error(ZSP_EINVAL, "schedule is NULL");
    if (!s->bound) return set_error(ZSP_ESTATE, "schedule has no arena (call zsp_sched_bind)");
    if (position != s->held || position < 0)
        return set_error(ZSP_ESTATE, "release of position %d, which is not held", position);
    if (s->depth > 0) {
        hipError_t e = hipEventRecord(s->mark, static_cast<hipStream_t>(compute_stream));
        if (e != hipSuccess) return zsp::set_hip_error(e, "hipEventRecord");
    }
    s->held = -1;
    s->next = position + 1;
    if (s->next == int32_t(s->order.size())) {
        s->next = 0;
        s->issued = -1;
    }
    return ZSP_OK;
}

zsp_status zsp_sched_set_engine(zsp_sched* s, zsp_gather_engine engine) {
    if (!s) return zsp::set_error(ZSP_EINVAL, "schedule is NULL");
    if (engine != ZSP_ENGINE_KERNEL && engine != ZSP_ENGINE_COPY)
        return zsp::set_error(ZSP_EINVAL, "bad gather engine %d", engine);
    if (s->held >= 0)
        return zsp::set_error(ZSP_ESTATE, "position %d is held", s->held);
    if (s->bound) {
        drop_events(s);
        s->bound = false;
    }
    s->engine = engine;
    return ZSP_OK;
}

zsp_status zsp_sched_reset(zsp_sched* s) {
    if (!s) return zsp::set_error(ZSP_EINVAL, "schedule is NULL");
    s->next = 0;
    s->held = -1;
    s->issued = -1;
    return ZSP_OK;
}

zsp_status zsp_sched_info(const zsp_sched* s, int32_t* depth, int32_t* slots,
                          int64_t* slot_bytes) {
    if (!s) return zsp::set_error(ZSP_EINVAL, "schedule is NULL");
    if (depth) *depth = s->depth;
    if (slots) *slots = s->slots;
    if (slot_bytes) *slot_bytes = s->slot_bytes;
    return ZSP_OK;
}

void zsp_sched_destroy(zsp_sched* s) {
    if (!s) return;
    drop_events(s);
    delete s;
}

}  // extern "C"
