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
#include <utility>

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

bool wants_span_table(const HostGatherTable& g) {
    return int64_t(g.delta.size()) * kShortPiece > g.total;
}

// Span building. Tiles are added to the current span in order while the
// span's tiles, runs, pieces and LDS chunks stay within the limits, and
// while each tile starts where the one before it ended; any other tile
// starts the next span. A rank's run is the range of its shard from the
// first to the last element the span reads from it; its LDS image starts at
// the 16-byte chunk holding the first element.
bool build_spans(const HostGatherTable& g, int64_t S, int32_t nd, const SpanTileIn* in,
                 int64_t n_in, int32_t max_tiles, SpanBuild& out) {
    out = SpanBuild{};
    const int64_t nq = static_cast<int64_t>(g.delta.size());
    if (n_in == 0) return true;
    if (S <= 0 || nd < 1 || nq == 0) return false;
    constexpr int64_t C = kSpanChunkElems;
    auto extent = [](int64_t l, int64_t h) { return (h + C - 1) / C - l / C; };
    auto rank_of = [&](int64_t q) { return (g.k0[size_t(q)] + g.delta[size_t(q)]) / S; };
    // the piece holding flat index K
    auto piece_of = [&](int64_t K) {
        return int64_t(std::upper_bound(g.k0.begin(), g.k0.end() - 1, K) - g.k0.begin()) - 1;
    };

    const size_t n_ranks = static_cast<size_t>(nd);
    std::vector<int64_t> lo(n_ranks), hi(n_ranks), stamp(n_ranks, -1);
    std::vector<int32_t> lds0(n_ranks), ranks;
    std::vector<std::pair<int64_t, int64_t>> segs;  // (piece, first global K in span)
    int64_t sid = 0, k_a = 0, chunks = 0, last_q = -1, next_K = -1;
    int32_t tiles = 0;
    struct TileRun {
        int64_t r, lo, hi;
    };
    std::vector<TileRun> trun;
    out.tile_segs.resize(static_cast<size_t>(n_in));

    auto finish = [&]() -> bool {
        std::sort(ranks.begin(), ranks.end());
        SpanRec rec{k_a, tiles, int32_t(ranks.size()), int32_t(out.runs.size()),
                    int32_t(out.segs.size()), int32_t(segs.size()), int32_t(chunks)};
        if (out.runs.size() + ranks.size() > size_t(INT32_MAX) ||
            out.segs.size() + segs.size() > size_t(INT32_MAX))
            return false;
        int32_t at = 0;
        for (int32_t r : ranks) {
            const int64_t c0 = lo[size_t(r)] / C;
            const int32_t n = int32_t(extent(lo[size_t(r)], hi[size_t(r)]));
            out.runs.push_back(SpanRun{c0, at, n});
            lds0[size_t(r)] = at;
            at += n;
        }
        for (const auto& sq : segs) {
            const int64_t q = sq.first, K = sq.second;
            const int64_t r = rank_of(q);
            const int64_t pos = C * lds0[size_t(r)] + (K + g.delta[size_t(q)] - C * (lo[size_t(r)] / C));
            const int64_t k = K - k_a;
            out.segs.push_back(SpanSeg{int32_t(k), int32_t(pos - k)});
        }
        out.spans.push_back(rec);
        ranks.clear();
        segs.clear();
        chunks = 0;
        tiles = 0;
        last_q = -1;
        ++sid;
        return true;
    };

    int64_t q_prev_last = -1;
    for (int64_t t = 0; t < n_in; ++t) {
        const int64_t t0 = in[t].K0, t1 = in[t].K0 + in[t].n;
        if (in[t].n <= 0 || t0 < 0 || t1 > g.total) return false;
        const bool joins = t0 == next_K;
        // first piece meeting the tile: walk on from the previous tile's
        // last piece when this tile follows it, else search
        int64_t q0 = joins ? q_prev_last : piece_of(t0);
        while (q0 + 1 < nq && g.k0[size_t(q0) + 1] <= t0) ++q0;
        int64_t q1 = q0;  // last piece meeting the tile
        while (q1 + 1 < nq && g.k0[size_t(q1) + 1] < t1) ++q1;
        q_prev_last = q1;
        // the tile's range of each rank (pieces of one rank merged)
        trun.clear();
        for (int64_t q = q0; q <= q1; ++q) {
            const int64_t a = std::max(g.k0[size_t(q)], t0) + g.delta[size_t(q)];
            const int64_t b = std::min(g.k0[size_t(q) + 1], t1) + g.delta[size_t(q)];
            const int64_t r = rank_of(q);
            bool merged = false;
            for (auto& x : trun) {
                if (x.r == r) {
                    x.lo = std::min(x.lo, a);
                    x.hi = std::max(x.hi, b);
                    merged = true;
                    break;
                }
            }
            if (!merged) trun.push_back(TileRun{r, a, b});
        }
        for (int pass = 0; pass < 2; ++pass) {
            int64_t add_chunks = 0, add_runs = 0;
            for (const auto& x : trun) {
                if (stamp[size_t(x.r)] == sid) {
                    const int64_t l = lo[size_t(x.r)], h = hi[size_t(x.r)];
                    add_chunks += extent(std::min(l, x.lo), std::max(h, x.hi)) - extent(l, h);
                } else {
                    add_chunks += extent(x.lo, x.hi);
                    ++add_runs;
                }
            }
            const bool cont = tiles > 0 && t0 == next_K;
            const int64_t add_segs = (q1 - q0 + 1) - (cont && q0 == last_q ? 1 : 0);
            const bool fits = (tiles == 0 || cont) && tiles + 1 <= max_tiles &&
                              chunks + add_chunks <= kSpanChunks &&
                              int64_t(segs.size()) + add_segs <= kSpanSegs &&
                              int64_t(ranks.size()) + add_runs <= kSpanRuns;
            if (fits) {
                for (const auto& x : trun) {
                    if (stamp[size_t(x.r)] == sid) {
                        lo[size_t(x.r)] = std::min(lo[size_t(x.r)], x.lo);
                        hi[size_t(x.r)] = std::max(hi[size_t(x.r)], x.hi);
                    } else {
                        stamp[size_t(x.r)] = sid;
                        lo[size_t(x.r)] = x.lo;
                        hi[size_t(x.r)] = x.hi;
                        ranks.push_back(int32_t(x.r));
                    }
                }
                chunks += add_chunks;
                if (tiles == 0) k_a = t0;
                const bool shares = cont && q0 == last_q;
                const uint32_t first = uint32_t(shares ? segs.size() - 1 : segs.size());
                for (int64_t q = q0; q <= q1; ++q) {
                    if (shares && q == q0) continue;
                    segs.emplace_back(q, std::max(g.k0[size_t(q)], t0));
                }
                last_q = q1;
                next_K = t1;
                out.tile_segs[size_t(t)] = first | (uint32_t(segs.size() - 1) << 16);
                ++tiles;
                break;
            }
            if (tiles == 0 || pass == 1) return false;  // the tile alone does not fit
            if (!finish()) return false;
        }
    }
    if (tiles > 0 && !finish()) return false;
    return true;
}

// Span tables of the range gather: spans of up to kSpanTiles tiles of the
// global 512-element grid, packed into 64-byte records.
void build_span_table(int64_t S, int32_t nd, HostGatherTable& g) {
    g.spans.clear();
    g.span_runs.clear();
    g.span_segs.clear();
    g.tile_segs.clear();
    g.wspans.clear();
    const int64_t total = g.total;
    if (total <= 0 || g.delta.empty()) return;
    const int64_t ntile = (total + kTile - 1) / kTile;
    std::vector<SpanTileIn> in(static_cast<size_t>(ntile));
    for (int64_t t = 0; t < ntile; ++t)
        in[size_t(t)] = SpanTileIn{t * kTile, std::min(kTile, total - t * kTile)};
    SpanBuild b;
    if (!build_spans(g, S, nd, in.data(), ntile, kSpanTiles, b)) return;
    g.spans = std::move(b.spans);
    g.span_runs = std::move(b.runs);
    g.span_segs = std::move(b.segs);
    g.tile_segs = std::move(b.tile_segs);
    auto fail = [&]() {
        g.spans.clear();
        g.span_runs.clear();
        g.span_segs.clear();
        g.tile_segs.clear();
        g.wspans.clear();
    };
    // device records: runs and per-tile pieces inline; a layout whose runs
    // lie more than 2^31 chunks apart, or with more than 2^31 tiles, gets none
    g.wspans.assign(g.spans.size(), WaveSpan{});
    for (size_t i = 0; i < g.spans.size(); ++i) {
        const SpanRec& R = g.spans[i];
        WaveSpan& w = g.wspans[i];
        if (R.k_a / kTile > INT32_MAX) {
            fail();
            return;
        }
        w.tile0 = int32_t(R.k_a / kTile);
        w.seg_first = R.seg_first;
        w.chunks = uint8_t(R.chunks);
        w.nrun = uint8_t(R.nrun);
        w.nseg = uint8_t(R.nseg);
        w.ntile = uint8_t(R.tiles);
        for (int32_t t = 0; t < R.tiles; ++t) {
            const uint32_t ts = g.tile_segs[size_t(R.k_a / kTile + t)];
            w.tseg[t] = uint16_t((ts & 0xffffu) | ((ts >> 16) << 8));
        }
        if (!pack_runs(g.span_runs.data() + R.run_first, R.nrun, w.chunk0, w.dchunk, w.lds0)) {
            fail();
            return;
        }
    }
}

bool pack_runs(const SpanRun* U, int32_t nrun, int64_t& chunk0, int32_t (&dchunk)[kSpanRuns - 1],
               uint8_t (&lds0)[kSpanRuns]) {
    chunk0 = U[0].chunk0;
    for (int32_t q = 0; q < kSpanRuns; ++q) {
        if (q < nrun) {
            lds0[q] = uint8_t(U[q].lds0);
            if (q > 0) {
                const int64_t d = U[q].chunk0 - U[0].chunk0;
                if (d > INT32_MAX || d < INT32_MIN) return false;
                dchunk[q - 1] = int32_t(d);
            }
        } else {
            lds0[q] = 0xffu;  // never reached by a chunk index
            if (q > 0) dchunk[q - 1] = 0;
        }
    }
    return true;
}

}  // namespace zsp
