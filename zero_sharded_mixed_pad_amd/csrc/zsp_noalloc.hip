// zsp_noalloc.hip -- zsp_gather_many_noalloc: zsp_gather_many for callers
// that cannot allocate. A long list's staging (its entries, coarse index and
// per-tile records) goes to `scratch`, a file-scope device array of fixed
// size that every GPU holds from library load to process end, instead of
// the plan's staging slots; nothing is allocated, on the host or the device.
//
// Host code never passes the array's name to a kernel or a copy (in host
// code it is a stand-in, not a device address): the array's address on each
// device is taken once, with that device current, by hipGetSymbolAddress
// (at an all-rank zsp_bind_state, or at this entry point's first call on a
// device), and that address is used from then on.
//
// One array per GPU serves every call on it: calls on one stream follow each
// other in order; calls on one GPU that overlap (other streams, other
// threads) race on it. Nothing in it needs clearing: a call writes every
// byte it reads before reading it. The staging copies read static host
// buffers that the next call refills, so a long list's call is not for
// stream capture (a replay would copy whatever those buffers hold then).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "zsp_entry.hpp"
#include "zsp_internal.hpp"
#include "zsp_list.hpp"
#include "zsp_plan.hpp"

namespace zsp {
namespace {

constexpr size_t kEntsMax = 65536;          // non-empty entries
constexpr size_t kCoarseMax = 65536;        // coarse slots: lists of up to 2^22 tiles
constexpr int64_t kRecTiles = int64_t(1) << 18;  // records per chunk
constexpr size_t kEntsBytes = kEntsMax * sizeof(ListEntry);         // 1 MiB
constexpr size_t kCoarseBytes = kCoarseMax * sizeof(int32_t);       // 256 KiB
constexpr size_t kRecBytes = size_t(kRecTiles) * sizeof(TileRec);   // 8 MiB
constexpr size_t kScratchBytes = kEntsBytes + kCoarseBytes + kRecBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Host staging: the entries and the coarse index are copied to the device
// in pieces through these two fixed buffers. hipMemcpyAsync from pageable
// memory has taken the bytes by the time it returns, so a buffer is
// refilled at once.
constexpr size_t kHostChunk = 32 * 1024;
ListEntry g_host_ents[kHostChunk / sizeof(ListEntry)];
int32_t g_host_coarse[kHostChunk / sizeof(int32_t)];
std::mutex g_host_mu;

// Collects consecutive values and copies each full buffer to dst.
template <typename V>
struct ChunkSink {
    V* buf;
    size_t cap;
    char* dst;
    hipStream_t stream;
    size_t first = 0, n = 0;
    hipError_t err = hipSuccess;
    void put(int64_t, const V& v) {
        buf[n++] = v;
        if (n == cap) flush();
    }
    void flush() {
        if (n > 0 && err == hipSuccess)
            err = hipMemcpyAsync(dst + first * sizeof(V), buf, n * sizeof(V),
                                 hipMemcpyHostToDevice, stream);
        first += n;
        n = 0;
    }
};

// The array's address on the current device (taken once per device).
zsp_status scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(ZSP_ERANGE, "device %d beyond the %d the library tracks", dev,
                         kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return set_hip_error(e, "hipGetSymbolAddress(scratch)");
        if (!p) return set_error(ZSP_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return ZSP_OK;
}

// Entries, then the coarse index, packed as the staged form lays them out
// and copied to the array at `d` (entries at 0, coarse index at kEntsBytes).
zsp_status upload(const zsp_plan* P, const int32_t* ids, int32_t n, void* const* outs,
                  char* d, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_host_mu);
    ChunkSink<ListEntry> es{g_host_ents, kHostChunk / sizeof(ListEntry), d, stream};
    ChunkSink<int32_t> cs{g_host_coarse, kHostChunk / sizeof(int32_t), d + kEntsBytes, stream};
    emit_staged(P, ids, n, outs, es, cs);
    es.flush();
    cs.flush();
    if (es.err != hipSuccess) return set_hip_error(es.err, "scratch staging copy");
    if (cs.err != hipSuccess) return set_hip_error(cs.err, "scratch staging copy");
    return ZSP_OK;
}

}  // namespace

// Takes the array's address on the current device ahead of the first call
// (an all-rank zsp_bind_state calls this).
zsp_status noalloc_setup() {
    void* p = nullptr;
    return scratch_ptr(&p);
}

}  // namespace zsp

extern "C" zsp_status zsp_gather_many_noalloc(zsp_plan* P, const int32_t* ids, int32_t n,
                                              zsp_source src, void* const* outs, void* stream) {
    using namespace zsp;
    ListTotals lt;
    zsp_status st = check_list(P, ids, n, src, outs, &lt);
    if (st != ZSP_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (lt.tiles == 0) return ZSP_OK;
    if (lt.count <= kListArgMax) return gather_list_args(P, ids, n, outs, src, lt, hs);
    if (size_t(lt.count) > kEntsMax)
        return set_error(ZSP_ERANGE,
                         "list of %lld non-empty parameters; this call stages at most %zu",
                         (long long)lt.count, kEntsMax);
    if (size_t((lt.tiles + 63) / 64) > kCoarseMax)
        return set_error(ZSP_ERANGE,
                         "list of %lld tiles of 512 elements; this call stages at most %zu",
                         (long long)lt.tiles, kCoarseMax * 64);
    void* base = nullptr;
    if ((st = scratch_ptr(&base)) != ZSP_OK) return st;
    char* d = static_cast<char*>(base);
    if ((st = upload(P, ids, n, outs, d, hs)) != ZSP_OK) return st;
    const StagedSizes z = staged_sizes(lt, kRecTiles);
    ListLaunch L = list_base(P, src, lt);
    L.ents = reinterpret_cast<const ListEntry*>(d);
    L.n_ents = static_cast<int32_t>(lt.count);
    L.coarse = reinterpret_cast<const int32_t*>(d + kEntsBytes);
    L.recs = reinterpret_cast<TileRec*>(d + kEntsBytes + kCoarseBytes);
    L.rec_cap = z.rec_tiles;
    return launch_list(L, src, hs);
}
