// zsp_gather_list.cpp -- zsp_gather_many: gather a list of parameters, in
// any order, each into its own output, in one pass ("The ZeRO-3 Diagram
// Most People Remember Is Wrong", section 3: a module's parameters are
// all-gathered just before it runs; section 8: gathers go out in buckets of
// parameters).
//
// A list of up to kListArgMax parameters with elements travels in the
// kernel arguments: one launch, nothing staged. A longer list is staged:
// its entries (output, parameter, first tile) and a coarse index (the entry
// of every 64th tile) are written to pinned host memory and copied to the
// device on the caller's stream; a first kernel turns them into one record
// per tile and a second copies the tiles. The plan keeps four staging
// slots, used in turn, each with an event recorded after its last kernel:
// a slot is refilled only once the work of its previous use has finished
// (the host waits for that event, which happens only with four staged
// gathers still in flight), so calls on any streams and threads stay
// apart. A slot grows, and is then reallocated, when a list needs more
// room than it has.
//
// A prepared list (zsp_gather_list_create) does the staged form's first
// kernel once: it keeps the records of every tile in device memory of its
// own, so each run is the copy kernel alone (a bucket gathered every step
// into the same outputs pays the staging once).
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "zsp_entry.hpp"
#include "zsp_internal.hpp"
#include "zsp_list.hpp"
#include "zsp_plan.hpp"

namespace zsp {

namespace {

constexpr int kSlots = 4;
// Tiles whose records one staged chunk holds (a multiple of 64): 16 MiB of
// records, 2^28 elements.
constexpr int64_t kRecChunk = int64_t(1) << 19;

struct ListSlot {
    void* host = nullptr;  // pinned: entries then coarse index
    size_t host_cap = 0;
    void* dev = nullptr;  // entries, coarse index, records
    size_t dev_cap = 0;
    hipEvent_t done = nullptr;
    bool pending = false;
};

size_t list_round_up(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

struct ListStaging {
    std::mutex mu;
    ListSlot slot[kSlots];
    int next = 0;
};

ListStaging* list_staging_new() { return new (std::nothrow) ListStaging(); }

void list_staging_free(ListStaging* ls) {
    if (!ls) return;
    for (ListSlot& s : ls->slot) {
        if (s.pending) (void)hipEventSynchronize(s.done);
        if (s.done) (void)hipEventDestroy(s.done);
        if (s.host) (void)hipHostFree(s.host);
        if (s.dev) (void)hipFree(s.dev);
    }
    delete ls;
}

zsp_status check_list(const zsp_plan* P, const int32_t* ids, int32_t n, zsp_source src,
                      void* const* outs, ListTotals* lt) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (P->bind_rank != ZSP_ALL_RANKS)
        return set_error(ZSP_ESTATE,
                         "gather needs every rank's shard (state bound for rank %d only)",
                         P->bind_rank);
    if (n < 0) return set_error(ZSP_EINVAL, "n = %d is negative", n);
    if (n > 0 && (!ids || !outs)) return set_error(ZSP_EINVAL, "ids or outs is NULL");
    if (src != ZSP_SRC_WORK && src != ZSP_SRC_MASTER && src != ZSP_SRC_ACC)
        return set_error(ZSP_EINVAL, "bad source %d", src);
    if (src == ZSP_SRC_ACC && !P->acc)
        return set_error(ZSP_ESTATE, "gather of the accumulator, but none is bound");
    int64_t count = 0, tiles = 0, elems = 0, pieces = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t t = ids[i];
        if (t < 0 || t >= P->T)
            return set_error(ZSP_ERANGE, "ids[%d] = %d outside [0, %d)", i, t, P->T);
        const int64_t numel = P->numel[size_t(t)];
        if (numel == 0) continue;
        if (!outs[i]) return set_error(ZSP_EINVAL, "outs[%d] is NULL", i);
        if (reinterpret_cast<uintptr_t>(outs[i]) & 15u)
            return set_error(ZSP_EINVAL, "outs[%d] is not 16-byte aligned", i);
        ++count;
        tiles += (numel + kTile - 1) / kTile;
        elems += numel;
        pieces += P->piece_off[size_t(t) + 1] - P->piece_off[size_t(t)];
        if (tiles > INT32_MAX)
            return set_error(ZSP_ERANGE, "list of more than 2^31 tiles of %lld elements",
                             (long long)kTile);
    }
    lt->count = count;
    lt->tiles = tiles;
    lt->short_pieces = pieces > 0 && elems < pieces * kShortPiece;
    return ZSP_OK;
}

ListLaunch list_base(const zsp_plan* P, zsp_source src, const ListTotals& lt) {
    ListLaunch L;
    L.params = P->params;
    L.S = P->S;
    L.src = src == ZSP_SRC_WORK     ? static_cast<const void*>(P->work)
            : src == ZSP_SRC_MASTER ? static_cast<const void*>(P->master)
                                    : static_cast<const void*>(P->acc);
    L.short_pieces = lt.short_pieces;
    L.tiles = lt.tiles;
    return L;
}

StagedSizes staged_sizes(const ListTotals& lt, int64_t rec_chunk) {
    StagedSizes z;
    z.ents = list_round_up(size_t(lt.count) * sizeof(ListEntry));
    z.coarse = list_round_up(size_t((lt.tiles + 63) / 64) * sizeof(int32_t));
    z.rec_tiles = std::min(rec_chunk, (lt.tiles + 63) / 64 * 64);
    z.recs = size_t(z.rec_tiles) * sizeof(TileRec);
    return z;
}

zsp_status launch_list(const ListLaunch& L, zsp_source src, hipStream_t stream) {
    const hipError_t e = launch_gather_list(L, src == ZSP_SRC_WORK ? 2 : 4, stream);
    if (e != hipSuccess) return set_hip_error(e, "list gather launch");
    return ZSP_OK;
}

ListLaunch list_args(const zsp_plan* P, const int32_t* ids, int32_t n, void* const* outs,
                     zsp_source src, const ListTotals& lt) {
    ListLaunch L = list_base(P, src, lt);
    L.n_args = static_cast<int32_t>(lt.count);
    for_each_entry(P, ids, n, outs,
                   [&](int64_t e, int32_t id, void* out, int64_t tile0, int64_t) {
                       const size_t t = size_t(id);
                       L.args[e] = ArgEntry{out, P->shard_off[t], P->shard_len[t], P->numel[t]};
                       L.arg_tile0[e] = static_cast<int32_t>(tile0);
                   });
    L.arg_tile0[L.n_args] = static_cast<int32_t>(lt.tiles);
    return L;
}

zsp_status gather_list_args(const zsp_plan* P, const int32_t* ids, int32_t n,
                            void* const* outs, zsp_source src, const ListTotals& lt,
                            hipStream_t stream) {
    return launch_list(list_args(P, ids, n, outs, src, lt), src, stream);
}

namespace {

// Writes the staged upload into one contiguous host buffer.
struct EntSink {
    ListEntry* p;
    void put(int64_t e, const ListEntry& v) { p[e] = v; }
};
struct CoarseSink {
    int32_t* p;
    void put(int64_t c, int32_t v) { p[c] = v; }
};

}  // namespace

}  // namespace zsp

extern "C" zsp_status zsp_gather_many(zsp_plan* P, const int32_t* ids, int32_t n,
                                      zsp_source src, void* const* outs, void* stream) {
    using namespace zsp;
    ListTotals lt;
    zsp_status st = check_list(P, ids, n, src, outs, &lt);
    if (st != ZSP_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (lt.tiles == 0) return ZSP_OK;
    if (lt.count <= kListArgMax) return gather_list_args(P, ids, n, outs, src, lt, hs);

    ListStaging& ls = *P->lists;  // made by the all-rank bind check_list asked for
    std::lock_guard<std::mutex> lock(ls.mu);
    ListSlot& s = ls.slot[ls.next];
    ls.next = (ls.next + 1) % kSlots;
    hipError_t e;
    if (s.pending) {
        if ((e = hipEventSynchronize(s.done)) != hipSuccess)
            return set_hip_error(e, "waiting for a staging slot");
        s.pending = false;
    }
    if (!s.done && (e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming)) != hipSuccess)
        return set_hip_error(e, "hipEventCreate");
    const StagedSizes z = staged_sizes(lt, kRecChunk);
    const size_t up = z.ents + z.coarse;
    if (s.host_cap < up) {
        if (s.host) (void)hipHostFree(s.host);
        s.host = nullptr;
        s.host_cap = 0;
        if ((e = hipHostMalloc(&s.host, up)) != hipSuccess)
            return set_error(ZSP_ENOMEM, "pinned staging of %zu bytes: %s", up,
                             hipGetErrorString(e));
        s.host_cap = up;
    }
    if (s.dev_cap < up + z.recs) {
        if (s.dev) (void)hipFree(s.dev);
        s.dev = nullptr;
        s.dev_cap = 0;
        if ((e = hipMalloc(&s.dev, up + z.recs)) != hipSuccess)
            return set_error(ZSP_ENOMEM, "device staging of %zu bytes: %s", up + z.recs,
                             hipGetErrorString(e));
        s.dev_cap = up + z.recs;
    }
    char* h = static_cast<char*>(s.host);
    EntSink es{reinterpret_cast<ListEntry*>(h)};
    CoarseSink cs{reinterpret_cast<int32_t*>(h + z.ents)};
    emit_staged(P, ids, n, outs, es, cs);
    ListLaunch L = list_base(P, src, lt);
    char* d = static_cast<char*>(s.dev);
    L.ents = reinterpret_cast<const ListEntry*>(d);
    L.n_ents = static_cast<int32_t>(lt.count);
    L.coarse = reinterpret_cast<const int32_t*>(d + z.ents);
    L.recs = reinterpret_cast<TileRec*>(d + up);
    L.rec_cap = z.rec_tiles;
    // the staging goes up through a kernel on the call's stream (up is a
    // multiple of 256 bytes; both buffers are 256-byte aligned)
    if ((e = launch_upload(s.dev, s.host, up, hs)) != hipSuccess)
        st = set_hip_error(e, "staging copy");
    else
        st = launch_list(L, src, hs);
    // Recorded even after a failed launch: the copy may be in flight.
    if ((e = hipEventRecord(s.done, hs)) != hipSuccess) {
        (void)hipStreamSynchronize(hs);
        return st != ZSP_OK ? st : set_hip_error(e, "hipEventRecord");
    }
    s.pending = true;
    return st;
}

// ---- Prepared lists ---------------------------------------------------------

struct zsp_gather_list {
    zsp_plan* plan = nullptr;
    zsp_source src = ZSP_SRC_WORK;
    int device = -1;
    zsp::ListLaunch L;    // argument form (n_args > 0) or records (mode 2)
    void* dev = nullptr;  // records form: entries, coarse index, records
};

extern "C" zsp_status zsp_gather_list_create(zsp_plan* P, const int32_t* ids, int32_t n,
                                             zsp_source src, void* const* outs, void* stream,
                                             zsp_gather_list** out) {
    using namespace zsp;
    if (!out) return set_error(ZSP_EINVAL, "out is NULL");
    *out = nullptr;
    ListTotals lt;
    zsp_status st = check_list(P, ids, n, src, outs, &lt);
    if (st != ZSP_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    zsp_gather_list* G = new (std::nothrow) zsp_gather_list();
    if (!G) return set_error(ZSP_ENOMEM, "out of host memory");
    G->plan = P;
    G->src = src;
    G->device = P->device;
    if (lt.tiles == 0) {
        G->L = list_base(P, src, lt);  // nothing to gather
    } else if (lt.count <= kListArgMax) {
        G->L = list_args(P, ids, n, outs, src, lt);
    } else {
        // Entries and coarse index made on the host, copied once; the
        // records of every tile are built on the device and kept.
        const StagedSizes z = staged_sizes(lt, INT64_MAX);
        const size_t up = z.ents + z.coarse;
        std::vector<char> host;
        try {
            host.assign(up, 0);
        } catch (const std::bad_alloc&) {
            delete G;
            return set_error(ZSP_ENOMEM, "out of host memory (%zu bytes)", up);
        }
        EntSink es{reinterpret_cast<ListEntry*>(host.data())};
        CoarseSink cs{reinterpret_cast<int32_t*>(host.data() + z.ents)};
        emit_staged(P, ids, n, outs, es, cs);
        hipError_t e = hipMalloc(&G->dev, up + z.recs);
        if (e != hipSuccess) {
            G->dev = nullptr;
            delete G;
            return set_error(ZSP_ENOMEM, "device list of %zu bytes: %s", up + z.recs,
                             hipGetErrorString(e));
        }
        ListLaunch L = list_base(P, src, lt);
        char* d = static_cast<char*>(G->dev);
        L.ents = reinterpret_cast<const ListEntry*>(d);
        L.n_ents = static_cast<int32_t>(lt.count);
        L.coarse = reinterpret_cast<const int32_t*>(d + z.ents);
        L.recs = reinterpret_cast<TileRec*>(d + up);
        L.rec_cap = z.rec_tiles;
        L.mode = 1;
        if ((e = hipMemcpyAsync(G->dev, host.data(), up, hipMemcpyHostToDevice, hs)) != hipSuccess)
            st = set_hip_error(e, "list copy");
        else
            st = launch_list(L, src, hs);
        // the host buffer, and the runs on any stream, wait for this work
        if ((e = hipStreamSynchronize(hs)) != hipSuccess && st == ZSP_OK)
            st = set_hip_error(e, "waiting for the list's records");
        if (st != ZSP_OK) {
            (void)hipFree(G->dev);
            delete G;
            return st;
        }
        L.mode = 2;
        G->L = L;
    }
    *out = G;
    return ZSP_OK;
}

extern "C" zsp_status zsp_gather_list_run(zsp_gather_list* G, void* stream) {
    using namespace zsp;
    if (!G) return set_error(ZSP_EINVAL, "list is NULL");
    const zsp_plan* P = G->plan;
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (P->bind_rank != ZSP_ALL_RANKS)
        return set_error(ZSP_ESTATE,
                         "gather needs every rank's shard (state bound for rank %d only)",
                         P->bind_rank);
    if (P->device != G->device)
        return set_error(ZSP_ESTATE, "list made on device %d, plan now bound on device %d",
                         G->device, P->device);
    if (G->src == ZSP_SRC_ACC && !P->acc)
        return set_error(ZSP_ESTATE, "gather of the accumulator, but none is bound");
    if (G->L.tiles == 0) return ZSP_OK;
    ListLaunch L = G->L;
    L.src = G->src == ZSP_SRC_WORK     ? static_cast<const void*>(P->work)
            : G->src == ZSP_SRC_MASTER ? static_cast<const void*>(P->master)
                                       : static_cast<const void*>(P->acc);
    return launch_list(L, G->src, static_cast<hipStream_t>(stream));
}

extern "C" void zsp_gather_list_destroy(zsp_gather_list* G) {
    if (!G) return;
    if (G->dev) (void)hipFree(G->dev);
    delete G;
}
