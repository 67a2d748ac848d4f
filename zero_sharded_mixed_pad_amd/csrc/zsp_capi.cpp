// zsp_capi.cpp -- the extern "C" entry points of libzsp (declared and
// documented in include/zsp.h): argument checks, plan bookkeeping, device
// table upload at bind time, and dispatch to the kernels.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "zsp_entry.hpp"
#include "zsp_internal.hpp"
#include "zsp_plan.hpp"

namespace {

thread_local std::string g_last_error;

zsp_status vfail(zsp_status st, const char* fmt, va_list ap) {
    char buf[512];
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    g_last_error = buf;
    return st;
}

zsp_status fail(zsp_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vfail(st, fmt, ap);
    va_end(ap);
    return st;
}

zsp_status fail_hip(hipError_t e, const char* what) {
    return fail(ZSP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

zsp_status check_device(const zsp_plan* P) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev != P->device)
        return fail(ZSP_ESTATE, "plan is bound on device %d but device %d is current", P->device,
                    dev);
    return ZSP_OK;
}

zsp_status check_bound(const zsp_plan* P) {
    if (!P) return fail(ZSP_EINVAL, "plan is NULL");
    if (!P->bound) return fail(ZSP_ESTATE, "no state bound (call zsp_bind_state first)");
    return check_device(P);
}

// E-space range of a rank-taking call.
zsp_status rank_range(const zsp_plan* P, int32_t rank, int64_t* b, int64_t* e) {
    if (P->bind_rank == ZSP_ALL_RANKS) {
        if (rank == ZSP_ALL_RANKS) {
            *b = 0;
            *e = int64_t(P->nd) * P->S;
            return ZSP_OK;
        }
        if (rank < 0 || rank >= P->nd)
            return fail(ZSP_EINVAL, "rank %d outside [0, %d) and not ZSP_ALL_RANKS", rank, P->nd);
        *b = int64_t(rank) * P->S;
        *e = *b + P->S;
        return ZSP_OK;
    }
    if (rank != P->bind_rank)
        return fail(ZSP_ESTATE, "state is bound for rank %d only, call named rank %d",
                    P->bind_rank, rank);
    *b = 0;
    *e = P->S;
    return ZSP_OK;
}

zsp_status check_grads(const zsp_plan* P, const void* const* grads, zsp_dtype dtype,
                       zsp_grad_layout layout) {
    if (dtype != ZSP_F32 && dtype != ZSP_BF16) return fail(ZSP_EINVAL, "bad dtype %d", dtype);
    if (layout != ZSP_GRADS_FULL && layout != ZSP_GRADS_SHARD)
        return fail(ZSP_EINVAL, "bad gradient layout %d", layout);
    if (!grads) return fail(ZSP_EINVAL, "grads array is NULL");
    for (int r = 0; r < P->nd; ++r) {
        if (!grads[r]) return fail(ZSP_EINVAL, "grads[%d] is NULL", r);
        if (!aligned16(grads[r])) return fail(ZSP_EINVAL, "grads[%d] is not 16-byte aligned", r);
    }
    return ZSP_OK;
}

// Elements of each gradient buffer the layout names.
int64_t grad_len(const zsp_plan* P, zsp_grad_layout layout) {
    if (layout == ZSP_GRADS_FULL) return P->total_padded;
    return P->bind_rank == ZSP_ALL_RANKS ? int64_t(P->nd) * P->S : P->S;
}

zsp_status adam_scalars(float lr, float b1, float b2, float eps, int64_t step,
                        zsp::AdamScalars* hp) {
    if (step < 1) return fail(ZSP_EINVAL, "step must be >= 1 (got %lld)", (long long)step);
    hp->lr = lr;
    hp->b1 = b1;
    hp->b2 = b2;
    hp->eps = eps;
    hp->omb1 = 1.0f - b1;
    hp->omb2 = 1.0f - b2;
    hp->bc1 = static_cast<float>(1.0 - std::pow(static_cast<double>(b1), static_cast<double>(step)));
    hp->bc2 = static_cast<float>(1.0 - std::pow(static_cast<double>(b2), static_cast<double>(step)));
    return ZSP_OK;
}

zsp::ShardLaunch base_launch(const zsp_plan* P) {
    zsp::ShardLaunch L;
    L.tab = P->shard;
    L.master = P->master;
    L.m = P->m;
    L.v = P->v;
    L.work = P->work;
    L.acc = P->acc;
    L.nd = P->nd;
    return L;
}

void free_tables(zsp_plan* P) {
    if (P->dev_blob) (void)hipFree(P->dev_blob);
    P->dev_blob = nullptr;
    P->shard = zsp::ShardTable{};
    P->gather = zsp::GatherTable{};
    P->span_k.clear();
    P->params = nullptr;
}

template <typename T>
size_t bytes_of(const std::vector<T>& v) {
    return v.size() * sizeof(T);
}

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

// Whether a shard launch over parameters [first, first + n) meets its pieces
// (one per rank and parameter with slots) every few thousand elements or
// less: such launches have many tiles at piece boundaries.
bool short_pieces(const zsp_plan* P, int32_t first, int32_t n) {
    const int64_t pieces = P->slot_off[size_t(first + n)] - P->slot_off[size_t(first)];
    const int64_t elems = P->shard_off[size_t(first + n)] - P->shard_off[size_t(first)];
    return pieces > 0 && elems < pieces * zsp::kShortPiece;
}

}  // namespace

namespace zsp {

zsp_status set_error(zsp_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vfail(st, fmt, ap);
    va_end(ap);
    return st;
}

zsp_status set_hip_error(hipError_t e, const char* what) { return fail_hip(e, what); }

zsp_status check_bound(const zsp_plan* P) { return ::check_bound(P); }

}  // namespace zsp

extern "C" {

zsp_status zsp_partition(const int64_t* numel, int32_t n_params, int32_t n_d, zsp_plan** out) {
    if (!out) return fail(ZSP_EINVAL, "out is NULL");
    *out = nullptr;
    if (!numel) return fail(ZSP_EINVAL, "numel is NULL");
    if (n_params < 1) return fail(ZSP_EINVAL, "n_params must be >= 1 (got %d)", n_params);
    if (n_d < 1 || n_d > ZSP_MAX_RANKS)
        return fail(ZSP_EINVAL, "n_d must be in [1, %d] (got %d)", ZSP_MAX_RANKS, n_d);
    zsp_plan* P = new (std::nothrow) zsp_plan();
    if (!P) return fail(ZSP_ENOMEM, "out of host memory");
    try {
        P->T = n_params;
        P->nd = n_d;
        P->numel.assign(numel, numel + n_params);
        P->pad.resize(n_params);
        P->shard_len.resize(n_params);
        P->full_off.assign(n_params + 1, 0);
        P->shard_off.assign(n_params + 1, 0);
        P->flat_off.assign(n_params + 1, 0);
        P->piece_off.assign(n_params + 1, 0);
        P->slot_off.assign(n_params + 1, 0);
        const int64_t kMax = int64_t(1) << 60;
        for (int32_t t = 0; t < n_params; ++t) {
            const int64_t n = numel[t];
            if (n < 0) {
                delete P;
                return fail(ZSP_EINVAL, "numel[%d] = %lld is negative", t, (long long)n);
            }
            if (n > kMax || P->full_off[t] > kMax - n - n_d) {
                delete P;
                return fail(ZSP_ERANGE, "total size exceeds 2^60 elements at parameter %d", t);
            }
            const int64_t pad = zsp::pad_for(n, n_d);
            P->pad[t] = pad;
            P->shard_len[t] = (n + pad) / n_d;
            P->full_off[t + 1] = P->full_off[t] + n + pad;
            P->shard_off[t + 1] = P->shard_off[t] + P->shard_len[t];
            P->flat_off[t + 1] = P->flat_off[t] + n;
            // ranks holding real elements of t: one gather piece each
            const int64_t s_t = P->shard_len[t];
            P->piece_off[t + 1] = P->piece_off[t] + (n == 0 ? 0 : (n + s_t - 1) / s_t);
            P->slot_off[t + 1] = P->slot_off[t] + (s_t > 0 ? 1 : 0);
        }
        P->S = P->shard_off[n_params];
        P->total_padded = P->full_off[n_params];
        P->total_numel = P->flat_off[n_params];
    } catch (const std::bad_alloc&) {
        delete P;
        return fail(ZSP_ENOMEM, "out of host memory");
    }
    *out = P;
    return ZSP_OK;
}

void zsp_destroy(zsp_plan* plan) {
    if (!plan) return;
    zsp::staging_free(plan->staging);
    zsp::list_staging_free(plan->lists);
    free_tables(plan);
    delete plan;
}

zsp_status zsp_plan_info(const zsp_plan* P, int64_t* shard_elems, int64_t* total_padded,
                         int64_t* model_state_bytes_per_rank) {
    if (!P) return fail(ZSP_EINVAL, "plan is NULL");
    if (shard_elems) *shard_elems = P->S;
    if (total_padded) *total_padded = P->total_padded;
    // 2 (16-bit param) + 2 (16-bit grad) + 4 (fp32 master) + 4 (m) + 4 (v)
    if (model_state_bytes_per_rank) *model_state_bytes_per_rank = 16 * P->S;
    return ZSP_OK;
}

zsp_status zsp_plan_tensor(const zsp_plan* P, int32_t t, int64_t* numel, int64_t* pad,
                           int64_t* shard_len, int64_t* full_off, int64_t* shard_off) {
    if (!P) return fail(ZSP_EINVAL, "plan is NULL");
    if (t < 0 || t >= P->T) return fail(ZSP_ERANGE, "parameter %d outside [0, %d)", t, P->T);
    if (numel) *numel = P->numel[t];
    if (pad) *pad = P->pad[t];
    if (shard_len) *shard_len = P->shard_len[t];
    if (full_off) *full_off = P->full_off[t];
    if (shard_off) *shard_off = P->shard_off[t];
    return ZSP_OK;
}

zsp_status zsp_bind_state(zsp_plan* P, int32_t rank_or_all, float* master, float* m, float* v,
                          uint16_t* work, float* grad_acc) {
    if (!P) return fail(ZSP_EINVAL, "plan is NULL");
    if (rank_or_all != ZSP_ALL_RANKS && (rank_or_all < 0 || rank_or_all >= P->nd))
        return fail(ZSP_EINVAL, "rank %d outside [0, %d) and not ZSP_ALL_RANKS", rank_or_all,
                    P->nd);
    const void* ptrs[4] = {master, m, v, work};
    const char* names[4] = {"master", "m", "v", "work"};
    for (int i = 0; i < 4; ++i) {
        if (!ptrs[i] && P->S > 0) return fail(ZSP_EINVAL, "%s is NULL", names[i]);
        if (!aligned16(ptrs[i])) return fail(ZSP_EINVAL, "%s is not 16-byte aligned", names[i]);
    }
    if (grad_acc && !aligned16(grad_acc))
        return fail(ZSP_EINVAL, "grad_acc is not 16-byte aligned");

    zsp::HostShardTable hs;
    zsp::HostGatherTable hg;
    std::vector<zsp::ParamInfo> hp;
    try {
        zsp::build_shard_table(P->numel, P->shard_len, P->full_off, P->shard_off, P->flat_off,
                               P->S, P->nd, rank_or_all, hs);
        if (rank_or_all == ZSP_ALL_RANKS) {
            zsp::build_gather_table(P->numel, P->shard_len, P->shard_off, P->flat_off, P->S,
                                    P->nd, hg);
            if (zsp::wants_span_table(hg)) zsp::build_span_table(P->S, P->nd, hg);
            hp.resize(size_t(P->T));
            for (int32_t t = 0; t < P->T; ++t)
                hp[size_t(t)] = zsp::ParamInfo{P->shard_off[size_t(t)], P->shard_len[size_t(t)],
                                               P->numel[size_t(t)], 0};
        }
    } catch (const std::bad_alloc&) {
        return fail(ZSP_ENOMEM, "out of host memory building tables");
    }
    if (hs.e0.size() > size_t(0x7fffffff) || hg.k0.size() > size_t(0x7fffffff))
        return fail(ZSP_ERANGE, "more than 2^31 pieces");

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");

    // One allocation: [e0 | info | tile | k0 | delta | gtile | gtile_delta |
    // gtile_pair | params | span records | span pieces], 256-byte aligned
    // parts.
    constexpr int kParts = 11;
    const size_t sz[kParts] = {bytes_of(hs.e0), bytes_of(hs.info),  bytes_of(hs.tile),
                               bytes_of(hg.k0), bytes_of(hg.delta), bytes_of(hg.tile),
                               bytes_of(hg.tile_delta), bytes_of(hg.tile_pair), bytes_of(hp),
                               bytes_of(hg.wspans), bytes_of(hg.span_segs)};
    const void* src[kParts] = {hs.e0.data(), hs.info.data(),  hs.tile.data(),
                               hg.k0.data(), hg.delta.data(), hg.tile.data(),
                               hg.tile_delta.data(), hg.tile_pair.data(), hp.data(),
                               hg.wspans.data(), hg.span_segs.data()};
    size_t off[kParts], total = 0;
    for (int i = 0; i < kParts; ++i) {
        off[i] = total;
        total += round_up(sz[i]);
    }
    free_tables(P);
    P->bound = false;
    void* blob = nullptr;
    if (total > 0) {
        e = hipMalloc(&blob, total);
        if (e != hipSuccess) return fail(ZSP_ENOMEM, "hipMalloc of %zu table bytes: %s", total,
                                         hipGetErrorString(e));
        for (int i = 0; i < kParts; ++i) {
            if (!sz[i]) continue;
            e = hipMemcpy(static_cast<char*>(blob) + off[i], src[i], sz[i],
                          hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                (void)hipFree(blob);
                return fail_hip(e, "hipMemcpy of offset tables");
            }
        }
    }
    if (P->lists && dev != P->device) {
        zsp::list_staging_free(P->lists);  // its slots live on the old device
        P->lists = nullptr;
    }
    if (rank_or_all == ZSP_ALL_RANKS && !P->lists) {
        P->lists = zsp::list_staging_new();
        if (!P->lists) {
            if (blob) (void)hipFree(blob);
            return fail(ZSP_ENOMEM, "out of host memory");
        }
    }
    if (rank_or_all == ZSP_ALL_RANKS) {
        // the no-alloc list gather's device array, located on this device now
        const zsp_status st = zsp::noalloc_setup();
        if (st != ZSP_OK) {
            if (blob) (void)hipFree(blob);
            return st;
        }
    }
    char* b = static_cast<char*>(blob);
    P->dev_blob = blob;
    P->shard.e0 = reinterpret_cast<const int64_t*>(b + off[0]);
    P->shard.info = reinterpret_cast<const zsp::PieceInfo*>(b + off[1]);
    P->shard.tile = reinterpret_cast<const int32_t*>(b + off[2]);
    P->shard.np = int64_t(hs.info.size());
    P->shard.ntile = hs.tile.empty() ? 0 : int64_t(hs.tile.size()) - 1;
    P->shard.total = hs.total;
    if (rank_or_all == ZSP_ALL_RANKS) {
        P->gather.k0 = reinterpret_cast<const int64_t*>(b + off[3]);
        P->gather.delta = reinterpret_cast<const int64_t*>(b + off[4]);
        P->gather.tile = reinterpret_cast<const int32_t*>(b + off[5]);
        P->gather.tile_delta = reinterpret_cast<const int64_t*>(b + off[6]);
        P->gather.tile_pair = reinterpret_cast<const int64_t*>(b + off[7]);
        P->gather.nq = int64_t(hg.delta.size());
        P->gather.ntile = hg.tile.empty() ? 0 : int64_t(hg.tile.size()) - 1;
        P->gather.total = hg.total;
        P->params = reinterpret_cast<const zsp::ParamInfo*>(b + off[8]);
        if (!hg.wspans.empty()) {
            P->gather.spans = reinterpret_cast<const zsp::WaveSpan*>(b + off[9]);
            P->gather.span_segs = reinterpret_cast<const zsp::SpanSeg*>(b + off[10]);
            P->gather.nspan = int64_t(hg.wspans.size());
            P->span_k.resize(hg.spans.size());
            for (size_t i = 0; i < hg.spans.size(); ++i) P->span_k[i] = hg.spans[i].k_a;
        }
    }
    P->bind_rank = rank_or_all;
    P->device = dev;
    P->master = master;
    P->m = m;
    P->v = v;
    P->work = work;
    P->acc = grad_acc;
    P->bound = true;
    return ZSP_OK;
}

zsp_status zsp_load_params(zsp_plan* P, const void* flat_params, zsp_dtype dtype, void* stream) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (dtype != ZSP_F32 && dtype != ZSP_BF16) return fail(ZSP_EINVAL, "bad dtype %d", dtype);
    if (!flat_params && P->total_numel > 0) return fail(ZSP_EINVAL, "flat_params is NULL");
    if (!aligned16(flat_params)) return fail(ZSP_EINVAL, "flat_params is not 16-byte aligned");
    zsp::ShardLaunch L = base_launch(P);
    L.e_begin = 0;
    L.e_end = P->shard.total;
    L.src = flat_params;
    L.short_pieces = short_pieces(P, 0, P->T);
    hipError_t e = zsp::launch_shard_op(L, zsp::OP_COPYIN, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, "copy-in launch");
    return ZSP_OK;
}

}  // extern "C"

namespace {

// The state spans a call on parameters [first, first + n) covers: for each
// rank it acts on, that rank's slots of those parameters, one contiguous
// span of the shard index space. Every parameter gives a single span over
// the whole bound range.
zsp_status param_spans(const zsp_plan* P, int32_t rank_or_all, int32_t first, int32_t n,
                       std::vector<std::pair<int64_t, int64_t>>* spans) {
    int64_t b, e;
    zsp_status st = rank_range(P, rank_or_all, &b, &e);
    if (st != ZSP_OK) return st;
    if (n < 1 || first < 0 || first > P->T - n)
        return fail(ZSP_ERANGE, "parameters [%d, %d+%d) outside [0, %d)", first, first, n, P->T);
    spans->clear();
    if (first == 0 && n == P->T) {
        spans->emplace_back(b, e);
        return ZSP_OK;
    }
    const int64_t lo = P->shard_off[size_t(first)], hi = P->shard_off[size_t(first + n)];
    for (int64_t base = b; base < e; base += P->S) spans->emplace_back(base + lo, base + hi);
    return ZSP_OK;
}

zsp_status launch_spans(zsp::ShardLaunch L, const std::vector<std::pair<int64_t, int64_t>>& spans,
                        zsp::ShardOp op, zsp_dtype dtype, void* stream, const char* what) {
    for (const auto& sp : spans) {
        L.e_begin = sp.first;
        L.e_end = sp.second;
        const hipError_t e = zsp::launch_shard_op(L, op, dtype, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail_hip(e, what);
    }
    return ZSP_OK;
}

zsp_status reduce_params(zsp_plan* P, int32_t rank_or_all, int32_t first, int32_t n,
                         const void* const* grads, zsp_dtype dtype, zsp_grad_layout layout,
                         int32_t accumulate, void* stream) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (!P->acc) return fail(ZSP_ESTATE, "reduce_shard needs a bound grad_acc");
    std::vector<std::pair<int64_t, int64_t>> spans;
    if ((st = param_spans(P, rank_or_all, first, n, &spans)) != ZSP_OK) return st;
    if ((st = check_grads(P, grads, dtype, layout)) != ZSP_OK) return st;
    zsp::ShardLaunch L = base_launch(P);
    L.grads = grads;
    L.shard_layout = layout == ZSP_GRADS_SHARD;
    L.grad_len = grad_len(P, layout);
    L.short_pieces = short_pieces(P, first, n);
    return launch_spans(L, spans, accumulate ? zsp::OP_REDUCE_ACC : zsp::OP_REDUCE_SET, dtype,
                        stream, "reduce launch");
}

zsp_status adam_params(zsp_plan* P, int32_t rank_or_all, int32_t first, int32_t n, float lr,
                       float beta1, float beta2, float eps, int64_t step, void* stream) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (!P->acc) return fail(ZSP_ESTATE, "adam_step reads grad_acc, which is not bound");
    std::vector<std::pair<int64_t, int64_t>> spans;
    if ((st = param_spans(P, rank_or_all, first, n, &spans)) != ZSP_OK) return st;
    zsp::ShardLaunch L = base_launch(P);
    if ((st = adam_scalars(lr, beta1, beta2, eps, step, &L.hp)) != ZSP_OK) return st;
    L.short_pieces = short_pieces(P, first, n);
    return launch_spans(L, spans, zsp::OP_ADAM, ZSP_F32, stream, "adam launch");
}

zsp_status reduce_adam_params(zsp_plan* P, int32_t rank_or_all, int32_t first, int32_t n,
                              const void* const* grads, zsp_dtype dtype, zsp_grad_layout layout,
                              int32_t use_acc, float lr, float beta1, float beta2, float eps,
                              int64_t step, void* stream) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (use_acc && !P->acc) return fail(ZSP_ESTATE, "use_acc needs a bound grad_acc");
    std::vector<std::pair<int64_t, int64_t>> spans;
    if ((st = param_spans(P, rank_or_all, first, n, &spans)) != ZSP_OK) return st;
    if ((st = check_grads(P, grads, dtype, layout)) != ZSP_OK) return st;
    zsp::ShardLaunch L = base_launch(P);
    if ((st = adam_scalars(lr, beta1, beta2, eps, step, &L.hp)) != ZSP_OK) return st;
    L.grads = grads;
    L.shard_layout = layout == ZSP_GRADS_SHARD;
    L.grad_len = grad_len(P, layout);
    L.short_pieces = short_pieces(P, first, n);
    return launch_spans(L, spans, use_acc ? zsp::OP_FUSED_ACC : zsp::OP_FUSED, dtype, stream,
                        "fused reduce+adam launch");
}

}  // namespace

extern "C" {

zsp_status zsp_reduce_shard(zsp_plan* P, int32_t rank_or_all, const void* const* grads,
                            zsp_dtype dtype, zsp_grad_layout layout, int32_t accumulate,
                            void* stream) {
    return reduce_params(P, rank_or_all, 0, P ? P->T : 0, grads, dtype, layout, accumulate,
                         stream);
}

zsp_status zsp_reduce_shard_params(zsp_plan* P, int32_t rank_or_all, int32_t first_param,
                                   int32_t n_params, const void* const* grads, zsp_dtype dtype,
                                   zsp_grad_layout layout, int32_t accumulate, void* stream) {
    return reduce_params(P, rank_or_all, first_param, n_params, grads, dtype, layout,
                         accumulate, stream);
}

zsp_status zsp_adam_step(zsp_plan* P, int32_t rank_or_all, float lr, float beta1, float beta2,
                         float eps, int64_t step, void* stream) {
    return adam_params(P, rank_or_all, 0, P ? P->T : 0, lr, beta1, beta2, eps, step, stream);
}

zsp_status zsp_adam_step_params(zsp_plan* P, int32_t rank_or_all, int32_t first_param,
                                int32_t n_params, float lr, float beta1, float beta2, float eps,
                                int64_t step, void* stream) {
    return adam_params(P, rank_or_all, first_param, n_params, lr, beta1, beta2, eps, step,
                       stream);
}

zsp_status zsp_reduce_adam_step(zsp_plan* P, int32_t rank_or_all, const void* const* grads,
                                zsp_dtype dtype, zsp_grad_layout layout, int32_t use_acc,
                                float lr, float beta1, float beta2, float eps, int64_t step,
                                void* stream) {
    return reduce_adam_params(P, rank_or_all, 0, P ? P->T : 0, grads, dtype, layout, use_acc,
                              lr, beta1, beta2, eps, step, stream);
}

zsp_status zsp_reduce_adam_step_params(zsp_plan* P, int32_t rank_or_all, int32_t first_param,
                                       int32_t n_params, const void* const* grads,
                                       zsp_dtype dtype, zsp_grad_layout layout, int32_t use_acc,
                                       float lr, float beta1, float beta2, float eps,
                                       int64_t step, void* stream) {
    return reduce_adam_params(P, rank_or_all, first_param, n_params, grads, dtype, layout,
                              use_acc, lr, beta1, beta2, eps, step, stream);
}

zsp_status zsp_gather_range(zsp_plan* P, int32_t first_param, int32_t n_params, zsp_source src,
                            void* out, void* stream) {
    return zsp::gather_range(P, first_param, n_params, src, out, static_cast<hipStream_t>(stream));
}

}  // extern "C"

zsp_status zsp::gather_range(zsp_plan* P, int32_t first_param, int32_t n_params, zsp_source src,
                             void* out, hipStream_t stream) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (P->bind_rank != ZSP_ALL_RANKS)
        return fail(ZSP_ESTATE, "gather needs every rank's shard (state bound for rank %d only)",
                    P->bind_rank);
    if (n_params < 1 || first_param < 0 || first_param > P->T - n_params)
        return fail(ZSP_ERANGE, "parameters [%d, %d+%d) outside [0, %d)", first_param,
                    first_param, n_params, P->T);
    if (src != ZSP_SRC_WORK && src != ZSP_SRC_MASTER && src != ZSP_SRC_ACC)
        return fail(ZSP_EINVAL, "bad source %d", src);
    if (src == ZSP_SRC_ACC && !P->acc)
        return fail(ZSP_ESTATE, "gather of the accumulator, but none is bound");
    const int64_t k_first = P->flat_off[first_param];
    const int64_t count = P->flat_off[first_param + n_params] - k_first;
    if (count > 0 && !out) return fail(ZSP_EINVAL, "out is NULL");
    if (!aligned16(out)) return fail(ZSP_EINVAL, "out is not 16-byte aligned");
    zsp::GatherLaunch L;
    L.tab = P->gather;
    L.k_first = k_first;
    L.count = count;
    L.src = src == ZSP_SRC_WORK     ? static_cast<const void*>(P->work)
            : src == ZSP_SRC_MASTER ? static_cast<const void*>(P->master)
                                    : static_cast<const void*>(P->acc);
    L.out = out;
    const int64_t pieces = P->piece_off[first_param + n_params] - P->piece_off[first_param];
    L.short_pieces = pieces > 0 && count < pieces * zsp::kShortPiece;
    if (k_first % zsp::kTile == 0 && P->gather.tile_delta) {
        L.tile_delta = P->gather.tile_delta + k_first / zsp::kTile;
        L.tile_pair = P->gather.tile_pair + 3 * (k_first / zsp::kTile);
    }
    if (src == ZSP_SRC_WORK && L.short_pieces && P->gather.spans && k_first % zsp::kTile == 0 &&
        count >= zsp::kSpanMinElems) {
        // spans holding the launch's first and last tiles
        const auto first = std::upper_bound(P->span_k.begin(), P->span_k.end(), k_first) - 1;
        const auto last =
            std::upper_bound(P->span_k.begin(), P->span_k.end(), k_first + count - 1) - 1;
        L.span_first = first - P->span_k.begin();
        L.nspan = last - first + 1;
        L.src_elems = int64_t(P->nd) * P->S;
    }
    hipError_t e = zsp::launch_gather(L, src == ZSP_SRC_WORK ? ZSP_BF16 : ZSP_F32, stream);
    if (e != hipSuccess) return fail_hip(e, "gather launch");
    return ZSP_OK;
}

extern "C" {

zsp_status zsp_gather(zsp_plan* P, int32_t param_id, zsp_source src, void* out, void* stream) {
    if (P && (param_id < 0 || param_id >= P->T))
        return fail(ZSP_ERANGE, "parameter %d outside [0, %d)", param_id, P->T);
    return zsp_gather_range(P, param_id, 1, src, out, stream);
}


const char* zsp_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
