// zsp_layout.cpp -- host-side tables of libzsp: per-parameter padding and
// offsets, and the piece/tile tables the kernels use to map a flat index to
// its parameter without searching the whole table.
//
// Partition rule ("The ZeRO-3 Diagram Most People Remember Is Wrong",
// section 2; "ZeRO Stages: Sharding Optimizer State, Gradients, and
// Parameters", "What stage 1 partitions"): each parameter is flattened,
// padded to a multiple of N_d on its own, and rank r owns the contiguous
// slice [r*s, (r+1)*s) of it.
#include <algorithm>

#include "zsp_internal.hpp"

namespace zsp {

int64_t pad_for(int64_t numel, int32_t nd) {
    const int64_t r = numel % nd;
    return r == 0 ? 0 : nd - r;
}

// tile[g] = index of the run containing element min(g*kTile, total-1), for
// g = 0 .. ceil(total/kTile). `starts` holds the run starts plus a final
// sentinel equal to total; runs are non-empty.
void build_tile_index(const std::vector<int64_t>& starts, int64_t total,
                      std::vector<int32_t>& tile) {
    tile.clear();
    if (total <= 0) return;
    const int64_t nruns = static_cast<int64_t>(starts.size()) - 1;
    const int64_t ntile = (total + kTile - 1) / kTile;
    tile.resize(ntile + 1);
    int64_t p = 0;
    for (int64_t g = 0; g <= ntile; ++g) {
        const int64_t x = std::min(g * kTile, total - 1);
        while (p + 1 < nruns && starts[p + 1] <= x) ++p;
        tile[g] = static_cast<int32_t>(p);
    }
}

// E-space pieces for an all-rank binding (rank r's shard at r*S) or for a
// one-rank binding of rank j (its shard at 0).
void build_shard_table(const std::vector<int64_t>& numel, const std::vector<int64_t>& shard_len,
                       const std::vector<int64_t>& full_off,
                       const std::vector<int64_t>& shard_off,
                       const std::vector<int64_t>& flat_off, int64_t S, int32_t nd,
                       int32_t rank_or_all, HostShardTable& out) {
    out.e0.clear();
    out.info.clear();
    const int32_t r_lo = rank_or_all == ZSP_ALL_RANKS ? 0 : rank_or_all;
    const int32_t r_hi = rank_or_all == ZSP_ALL_RANKS ? nd : rank_or_all + 1;
    const int64_t T = static_cast<int64_t>(numel.size());
    for (int32_t r = r_lo; r < r_hi; ++r) {
        const int64_t base = rank_or_all == ZSP_ALL_RANKS ? int64_t(r) * S : 0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t s = shard_len[t];
            if (s == 0) continue;
            const int64_t first = int64_t(r) * s;  // index in the padded tensor
            const int64_t valid = std::max<int64_t>(0, std::min<int64_t>(s, numel[t] - first));
            const int64_t e0 = base + shard_off[t];
            out.e0.push_back(e0);
            out.info.push_back(PieceInfo{e0 + valid, e0 + s, full_off[t] + first - e0,
                                         flat_off[t] + first - e0});
        }
    }
    out.total = rank_or_all == ZSP_ALL_RANKS ? int64_t(nd) * S : S;
    out.e0.push_back(out.total);
    build_tile_index(out.e0, out.total, out.tile);
}

// K-space pieces: parameter t, rank r covers flat indices
// [flat_off[t] + r*s, flat_off[t] + r*s + valid) and reads them from
// r*S + shard_off[t] onwards in the n_d*S shard arrays.
void build_gather_table(const std::vector<int64_t>& numel,
                        const std::vector<int64_t>& shard_len,
                        const std::vector<int64_t>& shard_off,
                        const std::vector<int64_t>& flat_off, int64_t S, int32_t nd,
                        HostGatherTable& out) {
    out.k0.clear();
    out.delta.clear();
    const int64_t T = static_cast<int64_t>(numel.size());
    for (int64_t t = 0; t < T; ++t) {
        const int64_t s = shard_len[t];
        for (int32_t r = 0; r < nd && s > 0; ++r) {
            const int64_t first = int64_t(r) * s;
            const int64_t valid = std::max<int64_t>(0, std::min<int64_t>(s, numel[t] - first));
            if (valid == 0) continue;
            const int64_t k0 = flat_off[t] + first;
            out.k0.push_back(k0);
            out.delta.push_back(int64_t(r) * S + shard_off[t] - k0);
        }
    }
    out.total = flat_off[T];
    out.k0.push_back(out.total);
    build_tile_index(out.k0, out.total, out.tile);
    // One lookup for a tile inside one piece: its piece's delta. A full tile
    // g lies in piece p = tile[g] when p's run reaches (g+1)*kTile.
    const int64_t ntile = out.tile.empty() ? 0 : int64_t(out.tile.size()) - 1;
    out.tile_delta.assign(size_t(ntile), kNoTileDelta);
    for (int64_t g = 0; g < ntile; ++g) {
        const int32_t p = out.tile[size_t(g)];
        if ((g + 1) * kTile <= out.k0[size_t(p) + 1]) out.tile_delta[size_t(g)] = out.delta[size_t(p)];
    }
    // Short-piece gathers: a tile within at most two pieces gets the second
    // piece's start and both deltas, one record instead of two lookups.
    out.tile_pair.assign(size_t(3 * ntile), 0);
    for (int64_t g = 0; g < ntile; ++g) {
        const int64_t p = out.tile[size_t(g)];
        const int64_t last = std::min((g + 1) * kTile, out.total) - 1;
        int64_t q = p;
        while (q - p < 2 && out.k0[size_t(q) + 1] <= last) ++q;
        int64_t* r = &out.tile_pair[size_t(3 * g)];
        if (q - p >= 2) {
            r[0] = kNoTileDelta;
        } else {
            r[0] = q > p ? out.k0[size_t(q)] : INT64_MAX;
            r[1] = out.delta[size_t(p)];
            r[2] = out.delta[size_t(q)];
        }
    }
}

}  // namespace zsp
