// zsp_list.hpp -- the host side of the list gathers shared by
// zsp_gather_list.cpp (zsp_gather_many, staged through the plan's slots)
// and zsp_noalloc.hip (zsp_gather_many_noalloc, staged through a static
// device array). Nothing here allocates: every pass reads the caller's
// ids[] and outs[] directly.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

#include "zsp.h"
#include "zsp_internal.hpp"
#include "zsp_plan.hpp"

namespace zsp {

// What the checks learned about a list: its entries with elements (the
// only ones a gather touches), its tiles, and which form it takes.
struct ListTotals {
    int64_t count = 0;  // entries with elements
    int64_t tiles = 0;
    bool short_pieces = false;
};

// Bytes of a staged list's parts: entries, coarse index (each rounded up to
// 256 bytes), and the record area of rec_tiles tiles.
struct StagedSizes {
    size_t ents, coarse, recs;
    int64_t rec_tiles;
};

// Argument checks (as zsp_gather_many documents them) and the list's totals.
zsp_status check_list(const zsp_plan* P, const int32_t* ids, int32_t n, zsp_source src,
                      void* const* outs, ListTotals* lt);
// A launch description with the plan's tables and the source filled in.
ListLaunch list_base(const zsp_plan* P, zsp_source src, const ListTotals& lt);
// Sizes of the staged form with records for at most rec_chunk tiles at once.
StagedSizes staged_sizes(const ListTotals& lt, int64_t rec_chunk);
// Launch, turning a HIP failure into ZSP_EHIP with a message.
zsp_status launch_list(const ListLaunch& L, zsp_source src, hipStream_t stream);
// The kernel-argument form (lists of at most kListArgMax entries with
// elements): its launch description, and that launch.
ListLaunch list_args(const zsp_plan* P, const int32_t* ids, int32_t n, void* const* outs,
                     zsp_source src, const ListTotals& lt);
zsp_status gather_list_args(const zsp_plan* P, const int32_t* ids, int32_t n,
                            void* const* outs, zsp_source src, const ListTotals& lt,
                            hipStream_t stream);

// Calls f(entry, id, out, tile0, tiles) for each entry with elements, in
// list order; entry counts from 0 over those entries only.
template <typename F>
void for_each_entry(const zsp_plan* P, const int32_t* ids, int32_t n, void* const* outs, F f) {
    int64_t e = 0, tile0 = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t numel = P->numel[size_t(ids[i])];
        if (numel == 0) continue;
        const int64_t tiles = (numel + kTile - 1) / kTile;
        f(e, ids[i], outs[i], tile0, tiles);
        ++e;
        tile0 += tiles;
    }
}

// The staged form's upload, produced in pieces: the entries (ListEntry) go
// to ents.put(entry, value) and the coarse index (the entry holding tile
// 64c, for every c) to coarse.put(c, value).
template <typename E, typename C>
void emit_staged(const zsp_plan* P, const int32_t* ids, int32_t n, void* const* outs, E& ents,
                 C& coarse) {
    for_each_entry(P, ids, n, outs,
                   [&](int64_t e, int32_t id, void* out, int64_t tile0, int64_t tiles) {
                       ents.put(e, ListEntry{out, id, static_cast<int32_t>(tile0)});
                       for (int64_t c = (tile0 + 63) / 64; 64 * c < tile0 + tiles; ++c)
                           coarse.put(c, static_cast<int32_t>(e));
                   });
}

}  // namespace zsp
