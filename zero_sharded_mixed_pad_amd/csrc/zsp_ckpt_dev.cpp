// zsp_ckpt_dev.cpp -- the checkpoint entry points ("ZeRO Stages: Sharding
// Optimizer State, Gradients, and Parameters", "Where the shards live and
// what happens on failure": each rank saves its own shard set; one lost rank
// is restored from its own file; a restart under another rank count
// reshuffles the shards; the safe point is between steps).
//
// Device state moves through up to 16 lanes, each with its own stream
// (default priority), two pinned chunks and two events, kept by the plan
// between calls. A lane handles one rank file at a time, and lanes run on
// separate host threads, so files are written or read in parallel:
//   save: the device-to-host copy of chunk k+1 runs while chunk k is
//         checksummed and written;
//   load: every file the load needs (the loaded ranks' own files, or all
//         of them under another rank count) is first read and checked whole
//         (header, parameter list, checksum, one common step), so a bad
//         checkpoint never touches device state; the checked files are then
//         mapped read-only and each of the plan's shards is cut from them
//         straight into the chunks, a chunk-sized window at a time, each
//         chunk copied host-to-device while the next is cut.
// The lanes' streams wait on an event taken on the caller's stream, so a
// save or load follows the work queued there before the call; both return
// after their copies are done.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "zsp_ckpt.hpp"
#include "zsp_entry.hpp"
#include "zsp_internal.hpp"
#include "zsp_plan.hpp"

namespace zsp {

namespace {

constexpr int kLanes = 16;                     // files in flight at once
constexpr size_t kChunk = size_t(16) << 20;    // bytes per pinned chunk

}  // namespace

struct Lane {
    hipStream_t stream = nullptr;
    void* buf[2] = {nullptr, nullptr};  // pinned host chunks
    hipEvent_t ev[2] = {nullptr, nullptr};
};

struct CkptStaging {
    int device = -1;
    hipEvent_t ready = nullptr;  // taken on the caller's stream at each call
    std::vector<Lane> lanes;
};

void staging_free(CkptStaging* st) {
    if (!st) return;
    for (Lane& l : st->lanes) {
        if (l.stream) (void)hipStreamSynchronize(l.stream);
        for (int i = 0; i < 2; ++i) {
            if (l.ev[i]) (void)hipEventDestroy(l.ev[i]);
            if (l.buf[i]) (void)hipHostFree(l.buf[i]);
        }
        if (l.stream) (void)hipStreamDestroy(l.stream);
    }
    if (st->ready) (void)hipEventDestroy(st->ready);
    delete st;
}

namespace {

// The plan's staging with at least n lanes on the plan's device.
zsp_status get_staging(zsp_plan* P, int n, CkptStaging** out) {
    if (P->staging && P->staging->device != P->device) {
        staging_free(P->staging);
        P->staging = nullptr;
    }
    if (!P->staging) {
        CkptStaging* st = new (std::nothrow) CkptStaging;
        if (!st) return set_error(ZSP_ENOMEM, "out of host memory");
        st->device = P->device;
        hipError_t e = hipEventCreateWithFlags(&st->ready, hipEventDisableTiming);
        if (e != hipSuccess) {
            delete st;
            return set_hip_error(e, "hipEventCreateWithFlags");
        }
        P->staging = st;
    }
    CkptStaging* st = P->staging;
    while (int(st->lanes.size()) < n) {
        Lane l;
        hipError_t e = hipStreamCreateWithFlags(&l.stream, hipStreamNonBlocking);
        for (int i = 0; i < 2 && e == hipSuccess; ++i) {
            e = hipHostMalloc(&l.buf[i], kChunk, hipHostMallocDefault);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&l.ev[i], hipEventDisableTiming);
        }
        if (e != hipSuccess) {
            for (int i = 0; i < 2; ++i) {
                if (l.ev[i]) (void)hipEventDestroy(l.ev[i]);
                if (l.buf[i]) (void)hipHostFree(l.buf[i]);
            }
            if (l.stream) (void)hipStreamDestroy(l.stream);
            return set_hip_error(e, "creating checkpoint staging (stream, pinned chunks)");
        }
        st->lanes.push_back(l);
    }
    *out = st;
    return ZSP_OK;
}

// Order lanes [0, n) after the work queued on the caller's stream.
zsp_status follow_caller(CkptStaging* st, int n, hipStream_t caller) {
    hipError_t e = hipEventRecord(st->ready, caller);
    for (int i = 0; i < n && e == hipSuccess; ++i)
        e = hipStreamWaitEvent(st->lanes[size_t(i)].stream, st->ready, 0);
    if (e != hipSuccess) return set_hip_error(e, "ordering after the caller's stream");
    return ZSP_OK;
}

std::string hip_text(hipError_t e, const char* what) {
    return std::string(what) + ": " + hipGetErrorString(e);
}

// Run job(i, lane, &message) for i in [0, n) on up to `lanes` threads (the
// calling thread is lane 0), each made current on `device` first unless it
// is negative (jobs that only touch files). The first failure stops further
// jobs; its status and message are reported in the calling thread.
template <typename Job>
zsp_status run_lanes(int n, int lanes, int device, Job job) {
    std::atomic<int> next{0};
    std::atomic<bool> stop{false};
    std::mutex mu;
    zsp_status first = ZSP_OK;
    std::string msg;
    auto worker = [&](int lane) {
        if (device >= 0 && hipSetDevice(device) != hipSuccess) {
            std::lock_guard<std::mutex> g(mu);
            if (first == ZSP_OK) first = ZSP_EHIP, msg = "hipSetDevice in a checkpoint thread";
            stop = true;
            return;
        }
        while (!stop) {
            const int i = next++;
            if (i >= n) break;
            zsp_status st = ZSP_OK;
            std::string m;
            try {
                st = job(i, lane, &m);
            } catch (const std::bad_alloc&) {
                st = ZSP_ENOMEM;
                m = "out of host memory in a checkpoint thread";
            }
            if (st != ZSP_OK) {
                std::lock_guard<std::mutex> g(mu);
                if (first == ZSP_OK) first = st, msg = m;
                stop = true;
            }
        }
    };
    std::vector<std::thread> threads;
    const int w = std::max(1, std::min(n, lanes));
    for (int l = 1; l < w; ++l) {
        try {
            threads.emplace_back(worker, l);
        } catch (...) {
            break;  // fewer threads: the others take more jobs
        }
    }
    worker(0);
    for (std::thread& t : threads) t.join();
    if (first != ZSP_OK) return set_error(first, "%s", msg.c_str());
    return ZSP_OK;
}

// One rank's device state (master, m, v, work at `base`) as a payload
// source: chunked device-to-host copies into the lane's pinned chunks; the
// copy of chunk k+1 is queued before chunk k is handed to the file side.
class DevSource : public PayloadSource {
  public:
    DevSource(Lane& lane, const zsp_plan* P, int64_t base) : lane_(lane) {
        src_[0] = reinterpret_cast<const char*>(P->master + base);
        src_[1] = reinterpret_cast<const char*>(P->m + base);
        src_[2] = reinterpret_cast<const char*>(P->v + base);
        src_[3] = reinterpret_cast<const char*>(P->work + base);
        for (int i = 0; i < 4; ++i) len_[i] = size_t(P->S) * (i < 3 ? 4 : 2);
    }
    bool next(const void** data, size_t* n, std::string* err) override {
        if (issued_ == 0 && !issue(err)) return false;
        if (consumed_ == issued_) {
            *n = 0;
            return true;
        }
        if (!issue(err)) return false;  // the chunk after this one, into the other buffer
        const int b = consumed_ % 2;
        const hipError_t e = hipEventSynchronize(lane_.ev[b]);
        if (e != hipSuccess) {
            *err = hip_text(e, "device-to-host copy");
            return false;
        }
        *data = lane_.buf[b];
        *n = size_[b];
        ++consumed_;
        return true;
    }

  private:
    bool issue(std::string* err) {
        while (seg_ < 4 && off_ == len_[seg_]) {
            ++seg_;
            off_ = 0;
        }
        if (seg_ == 4) return true;  // nothing left to queue
        const int b = issued_ % 2;
        const size_t n = std::min(kChunk, len_[seg_] - off_);
        hipError_t e = hipMemcpyAsync(lane_.buf[b], src_[seg_] + off_, n, hipMemcpyDeviceToHost,
                                      lane_.stream);
        if (e == hipSuccess) e = hipEventRecord(lane_.ev[b], lane_.stream);
        if (e != hipSuccess) {
            *err = hip_text(e, "device-to-host copy");
            return false;
        }
        size_[b] = n;
        off_ += n;
        ++issued_;
        return true;
    }

    Lane& lane_;
    const char* src_[4];
    size_t len_[4];
    int seg_ = 0;
    size_t off_ = 0;
    size_t size_[2] = {0, 0};
    int issued_ = 0, consumed_ = 0;
};

// One rank's device state filled through the lane's pinned chunks: the
// caller writes a chunk, which is then copied host-to-device; a chunk is
// handed out again only once its previous copy has finished. The state is
// filled in payload order (master, m, v, work), each array whole.
class DevSink {
  public:
    DevSink(Lane& lane, const zsp_plan* P, int64_t base) : lane_(lane) {
        dst_[0] = reinterpret_cast<char*>(P->master + base);
        dst_[1] = reinterpret_cast<char*>(P->m + base);
        dst_[2] = reinterpret_cast<char*>(P->v + base);
        dst_[3] = reinterpret_cast<char*>(P->work + base);
        for (int i = 0; i < 4; ++i) len_[i] = size_t(P->S) * (i < 3 ? 4 : 2);
    }
    // A chunk for the next bytes, at most *cap of them (never past an array).
    bool buffer(void** data, size_t* cap, std::string* err) {
        while (seg_ < 4 && off_ == len_[seg_]) {
            ++seg_;
            off_ = 0;
        }
        if (seg_ == 4) {
            *err = "payload longer than the state";
            return false;
        }
        const int b = k_ % 2;
        if (used_[b]) {
            const hipError_t e = hipEventSynchronize(lane_.ev[b]);
            if (e != hipSuccess) {
                *err = hip_text(e, "host-to-device copy");
                return false;
            }
        }
        *data = lane_.buf[b];
        *cap = std::min(kChunk, len_[seg_] - off_);
        return true;
    }
    // The chunk last handed out now holds the next n bytes.
    bool commit(size_t n, std::string* err) {
        const int b = k_ % 2;
        hipError_t e = hipMemcpyAsync(dst_[seg_] + off_, lane_.buf[b], n, hipMemcpyHostToDevice,
                                      lane_.stream);
        if (e == hipSuccess) e = hipEventRecord(lane_.ev[b], lane_.stream);
        if (e != hipSuccess) {
            *err = hip_text(e, "host-to-device copy");
            return false;
        }
        used_[b] = true;
        off_ += n;
        ++k_;
        return true;
    }

  private:
    Lane& lane_;
    char* dst_[4];
    size_t len_[4];
    int seg_ = 0;
    size_t off_ = 0;
    int k_ = 0;
    bool used_[2] = {false, false};
};

// ---- rank layouts and resharding -------------------------------------------


struct RankLayout {
    std::vector<int64_t> shard_len, shard_off;
    int64_t S = 0;
};

RankLayout rank_layout(const std::vector<int64_t>& numel, int32_t nd) {
    RankLayout L;
    L.shard_len.resize(numel.size());
    L.shard_off.assign(numel.size() + 1, 0);
    for (size_t t = 0; t < numel.size(); ++t) {
        L.shard_len[t] = (numel[t] + pad_for(numel[t], nd)) / nd;
        L.shard_off[t + 1] = L.shard_off[t] + L.shard_len[t];
    }
    L.S = L.shard_off.back();
    return L;
}

// Checks shared by every read: the file's parameter list is the plan's and
// its S is the one the rank count gives.
bool same_model(const zsp_plan* P, const std::vector<int64_t>& numel, int64_t S, int64_t S_want) {
    return numel == P->numel && S == S_want;
}

// The files of a checkpoint that a load needs: each mapped read-only once and
// checked whole on that mapping (one lane per file), so that the plan's
// shards are cut from the page cache, from exactly the bytes the checksum
// covered, without another copy. Under the plan's own rank count a shard
// is one old file's payload; under another, it takes runs of every file.
struct OldCheckpoint {
    int32_t nd = 0;
    RankLayout L;
    std::vector<std::unique_ptr<MappedRank>> files;
    std::vector<const float*> master, m, v;
    std::vector<const uint16_t*> work;
};

// Check and map the files of the old ranks that the plan's ranks `ranks`
// need (all of them under another rank count); the others stay unmapped.
// The checked files must hold the plan's parameter list and one step.
zsp_status open_old(const zsp_plan* P, const char* dir, int32_t nd_old,
                    const std::vector<int32_t>& ranks, OldCheckpoint* old, int64_t* step) {
    old->nd = nd_old;
    old->L = rank_layout(P->numel, nd_old);
    std::vector<int32_t> need;
    if (nd_old == P->nd) {
        need = ranks;
    } else {
        for (int32_t r = 0; r < nd_old; ++r) need.push_back(r);
    }
    const int n = int(need.size());
    std::vector<int64_t> steps(size_t(n), 0);
    std::vector<std::unique_ptr<MappedRank>> opened(static_cast<size_t>(n));
    zsp_status st = run_lanes(n, kLanes, -1, [&](int i, int, std::string* m) {
        std::unique_ptr<MappedRank> f(new MappedRank);
        std::vector<int64_t> numel;
        int64_t S = 0;
        if (f->open(dir, nd_old, need[size_t(i)], &numel, &S, &steps[size_t(i)], m) !=
            CkptStatus::Ok)
            return ZSP_EIO;
        if (!same_model(P, numel, S, old->L.S)) {
            *m = std::string("checkpoint in ") + dir + " holds another parameter list";
            return ZSP_EIO;
        }
        opened[size_t(i)] = std::move(f);
        return ZSP_OK;
    });
    if (st != ZSP_OK) return st;
    for (int i = 1; i < n; ++i)
        if (steps[size_t(i)] != steps[0])
            return set_error(ZSP_EIO, "checkpoint in %s mixes steps %lld and %lld", dir,
                             (long long)steps[0], (long long)steps[size_t(i)]);
    *step = n > 0 ? steps[0] : 0;
    old->files.resize(size_t(nd_old));
    old->master.assign(size_t(nd_old), nullptr);
    old->m.assign(size_t(nd_old), nullptr);
    old->v.assign(size_t(nd_old), nullptr);
    old->work.assign(size_t(nd_old), nullptr);
    for (int i = 0; i < n; ++i) {
        const size_t r = size_t(need[size_t(i)]);
        MappedRank* f = opened[size_t(i)].get();
        old->master[r] = f->master();
        old->m[r] = f->m();
        old->v[r] = f->v();
        old->work[r] = f->work();
        old->files[r] = std::move(opened[size_t(i)]);
    }
    return ZSP_OK;
}

// Elements [e_lo, e_hi) of rank j's shard array under the plan's layout,
// cut from the old ranks' arrays: element k of parameter t lives in old
// rank k / s_old at k - r*s_old of its slice; pads are +0.
template <typename T>
void reshard_range(const zsp_plan* P, const RankLayout& Lo, int32_t j,
                   const std::vector<const T*>& old, int64_t e_lo, int64_t e_hi, T* out) {
    // last parameter starting at or before e_lo
    int32_t t = int32_t(std::upper_bound(P->shard_off.begin(), P->shard_off.end(), e_lo) -
                        P->shard_off.begin()) - 1;
    for (t = std::max(t, 0); t < P->T && P->shard_off[size_t(t)] < e_hi; ++t) {
        const int64_t s = P->shard_len[size_t(t)], so = Lo.shard_len[size_t(t)];
        const int64_t off = P->shard_off[size_t(t)];
        const int64_t i0 = std::max(e_lo, off) - off, i1 = std::min(e_hi, off + s) - off;
        if (i0 >= i1) continue;
        T* dst = out + (off + i0 - e_lo);
        int64_t k = int64_t(j) * s + i0;
        const int64_t k_slot_end = int64_t(j) * s + i1;
        const int64_t kend = std::min<int64_t>(P->numel[size_t(t)], k_slot_end);
        while (k < kend) {
            const int64_t r = k / so;
            const int64_t run_end = std::min<int64_t>(kend, (r + 1) * so);
            std::memcpy(dst, old[size_t(r)] + Lo.shard_off[size_t(t)] + (k - r * so),
                        size_t(run_end - k) * sizeof(T));
            dst += run_end - k;
            k = run_end;
        }
        if (k < k_slot_end) std::memset(dst, 0, size_t(k_slot_end - k) * sizeof(T));
    }
}

// Ranks a save/load call covers under the plan's binding.
zsp_status ckpt_ranks(const zsp_plan* P, int32_t rank_or_all, std::vector<int32_t>* ranks) {
    ranks->clear();
    if (P->bind_rank != ZSP_ALL_RANKS) {
        if (rank_or_all != ZSP_ALL_RANKS && rank_or_all != P->bind_rank)
            return set_error(ZSP_ESTATE, "state is bound for rank %d only, call named rank %d",
                             P->bind_rank, rank_or_all);
        ranks->push_back(P->bind_rank);
        return ZSP_OK;
    }
    if (rank_or_all == ZSP_ALL_RANKS) {
        for (int32_t r = 0; r < P->nd; ++r) ranks->push_back(r);
        return ZSP_OK;
    }
    if (rank_or_all < 0 || rank_or_all >= P->nd)
        return set_error(ZSP_EINVAL, "rank %d outside [0, %d) and not ZSP_ALL_RANKS",
                         rank_or_all, P->nd);
    ranks->push_back(rank_or_all);
    return ZSP_OK;
}

int64_t rank_base(const zsp_plan* P, int32_t r) {
    return P->bind_rank == ZSP_ALL_RANKS ? int64_t(r) * P->S : 0;
}

zsp_status find_checkpoint(const char* dir, int32_t* nd_old) {
    *nd_old = ckpt_find_nd(dir);
    if (*nd_old == 0)
        return set_error(ZSP_EIO, "no checkpoint (rank-<r>-of-<n>.zsp) in %s", dir);
    if (*nd_old < 0) return set_error(ZSP_EIO, "%s holds shard files of several rank counts", dir);
    return ZSP_OK;
}

}  // namespace
}  // namespace zsp

using namespace zsp;

extern "C" {

zsp_status zsp_checkpoint_write_host(const zsp_plan* P, int32_t rank, const char* dir,
                                     int64_t step, const float* master, const float* m,
                                     const float* v, const uint16_t* work) {
    if (!P) return set_error(ZSP_EINVAL, "plan is NULL");
    if (!dir) return set_error(ZSP_EINVAL, "dir is NULL");
    if (rank < 0 || rank >= P->nd)
        return set_error(ZSP_EINVAL, "rank %d outside [0, %d)", rank, P->nd);
    if (P->S > 0 && (!master || !m || !v || !work))
        return set_error(ZSP_EINVAL, "state arrays must not be NULL");
    HostPayload src(master, m, v, work, P->S);
    std::string err;
    if (ckpt_write_rank(dir, P->nd, rank, P->numel, P->S, step, src, &err) != CkptStatus::Ok)
        return set_error(ZSP_EIO, "%s", err.c_str());
    return ZSP_OK;
}

zsp_status zsp_checkpoint_read_host(const zsp_plan* P, int32_t rank, const char* dir,
                                    int64_t* step, float* master, float* m, float* v,
                                    uint16_t* work) {
    if (!P) return set_error(ZSP_EINVAL, "plan is NULL");
    if (!dir || !step) return set_error(ZSP_EINVAL, "dir and step must not be NULL");
    if (rank < 0 || rank >= P->nd)
        return set_error(ZSP_EINVAL, "rank %d outside [0, %d)", rank, P->nd);
    if (P->S > 0 && (!master || !m || !v || !work))
        return set_error(ZSP_EINVAL, "state arrays must not be NULL");
    int32_t nd_old = 0;
    zsp_status st = find_checkpoint(dir, &nd_old);
    if (st != ZSP_OK) return st;
    try {
        OldCheckpoint old;
        if ((st = open_old(P, dir, nd_old, std::vector<int32_t>{rank}, &old, step)) != ZSP_OK)
            return st;
        reshard_range(P, old.L, rank, old.master, 0, P->S, master);
        reshard_range(P, old.L, rank, old.m, 0, P->S, m);
        reshard_range(P, old.L, rank, old.v, 0, P->S, v);
        reshard_range(P, old.L, rank, old.work, 0, P->S, work);
    } catch (const std::bad_alloc&) {
        return set_error(ZSP_ENOMEM, "out of host memory reading the checkpoint");
    }
    return ZSP_OK;
}

zsp_status zsp_checkpoint_save(zsp_plan* P, int32_t rank_or_all, const char* dir, int64_t step,
                               void* stream) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (!dir) return set_error(ZSP_EINVAL, "dir is NULL");
    std::vector<int32_t> ranks;
    if ((st = ckpt_ranks(P, rank_or_all, &ranks)) != ZSP_OK) return st;
    const int lanes = std::min<int>(int(ranks.size()), kLanes);
    CkptStaging* stg = nullptr;
    if ((st = get_staging(P, lanes, &stg)) != ZSP_OK) return st;
    if ((st = follow_caller(stg, lanes, static_cast<hipStream_t>(stream))) != ZSP_OK) return st;
    return run_lanes(int(ranks.size()), lanes, P->device, [&](int i, int lane, std::string* m) {
        Lane& L = stg->lanes[size_t(lane)];
        const int32_t r = ranks[size_t(i)];
        DevSource src(L, P, rank_base(P, r));
        const CkptStatus cs = ckpt_write_rank(dir, P->nd, r, P->numel, P->S, step, src, m);
        const hipError_t e = hipStreamSynchronize(L.stream);  // no copy outlives the job
        if (cs != CkptStatus::Ok) return ZSP_EIO;
        if (e != hipSuccess) {
            *m = hip_text(e, "device-to-host copy");
            return ZSP_EHIP;
        }
        return ZSP_OK;
    });
}

zsp_status zsp_checkpoint_load(zsp_plan* P, int32_t rank_or_all, const char* dir, int64_t* step,
                               void* stream) {
    zsp_status st = check_bound(P);
    if (st != ZSP_OK) return st;
    if (!dir || !step) return set_error(ZSP_EINVAL, "dir and step must not be NULL");
    std::vector<int32_t> ranks;
    if ((st = ckpt_ranks(P, rank_or_all, &ranks)) != ZSP_OK) return st;
    int32_t nd_old = 0;
    if ((st = find_checkpoint(dir, &nd_old)) != ZSP_OK) return st;
    const int n = int(ranks.size());
    const int lanes = std::min<int>(n, kLanes);
    CkptStaging* stg = nullptr;
    if ((st = get_staging(P, lanes, &stg)) != ZSP_OK) return st;
    try {
        // check and map the files needed, then cut each of the plan's shards
        // into the pinned chunks, a chunk at a time
        OldCheckpoint old;
        if ((st = open_old(P, dir, nd_old, ranks, &old, step)) != ZSP_OK) return st;
        if ((st = follow_caller(stg, lanes, static_cast<hipStream_t>(stream))) != ZSP_OK)
            return st;
        return run_lanes(n, lanes, P->device, [&](int i, int lane, std::string* m) {
            Lane& L = stg->lanes[size_t(lane)];
            const int32_t r = ranks[size_t(i)];
            DevSink sink(L, P, rank_base(P, r));
            bool ok = true;
            for (int a = 0; a < 4 && ok; ++a) {  // master, m, v, work: payload order
                const size_t esz = a < 3 ? sizeof(float) : sizeof(uint16_t);
                for (int64_t e = 0; ok && e < P->S;) {
                    void* buf = nullptr;
                    size_t cap = 0;
                    ok = sink.buffer(&buf, &cap, m);
                    if (!ok) break;
                    const int64_t cnt = int64_t(cap / esz);
                    if (a == 0) reshard_range(P, old.L, r, old.master, e, e + cnt, (float*)buf);
                    if (a == 1) reshard_range(P, old.L, r, old.m, e, e + cnt, (float*)buf);
                    if (a == 2) reshard_range(P, old.L, r, old.v, e, e + cnt, (float*)buf);
                    if (a == 3) reshard_range(P, old.L, r, old.work, e, e + cnt, (uint16_t*)buf);
                    ok = sink.commit(size_t(cnt) * esz, m);
                    e += cnt;
                }
            }
            const hipError_t e = hipStreamSynchronize(L.stream);
            if (!ok) return ZSP_EHIP;
            if (e != hipSuccess) {
                *m = hip_text(e, "host-to-device copy");
                return ZSP_EHIP;
            }
            return ZSP_OK;
        });
    } catch (const std::bad_alloc&) {
        return set_error(ZSP_ENOMEM, "out of host memory reading the checkpoint");
    }
}

}  // extern "C"
